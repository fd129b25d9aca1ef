"""Pins of the prefill oracle (oracle/prefill.py) against facts outside it:
closed cases of causal softmax attention, causality, and the decode oracle's
dense attention (a separate C implementation) on the last row."""
from __future__ import annotations

import numpy as np

import oracle
from hash_top_sparse_amd import synth
from oracle import prefill

RNG = np.random.default_rng(4242)


def _gauss(shape):
    return synth.bf16_bits(RNG.standard_normal(shape).astype(np.float32))


def test_first_row_is_first_value_row():
    B, Hq, Hkv, S, d = 2, 4, 2, 9, 16
    q, K, V = _gauss((B, Hq, S, d)), _gauss((B, Hkv, S, d)), _gauss((B, Hkv, S, d))
    out = prefill.causal_attention(q, K, V, np.array([9, 5]))
    Vf = synth.bf16_to_f32(V).astype(np.float64)
    for b in range(B):
        for h in range(Hq):
            np.testing.assert_array_equal(out[b, h, 0], Vf[b, h // 2, 0])


def test_equal_logits_give_running_mean():
    B, Hq, Hkv, S, d = 1, 2, 1, 40, 8
    q = synth.bf16_bits(np.zeros((B, Hq, S, d), np.float32))
    K, V = _gauss((B, Hkv, S, d)), _gauss((B, Hkv, S, d))
    out = prefill.causal_attention(q, K, V, np.array([S]))
    Vf = synth.bf16_to_f32(V[0, 0]).astype(np.float64)
    want = np.cumsum(Vf, axis=0) / np.arange(1, S + 1)[:, None]
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], want, rtol=1e-12, atol=1e-12)


def test_dominant_logit_selects_its_value_row():
    S, d = 12, 16
    K = np.zeros((1, 1, S, d), np.float32)
    K[0, 0, :, 0] = np.arange(S)                # logit grows with the key index
    q = np.zeros((1, 1, S, d), np.float32)
    q[0, 0, :, 0] = 64.0                        # gap of 64 * scale = 16 per step
    V = RNG.standard_normal((1, 1, S, d)).astype(np.float32)
    out = prefill.causal_attention(synth.bf16_bits(q), synth.bf16_bits(K), synth.bf16_bits(V), [S], scale=0.25)
    Vf = synth.bf16_to_f32(synth.bf16_bits(V))[0, 0]
    for i in range(S):  # row i sees keys 0..i, key i dominates (weight >= 1 - 2e-7)
        np.testing.assert_allclose(out[0, 0, i], Vf[i], atol=1e-5 * max(1.0, np.abs(Vf).max()))


def test_later_keys_do_not_change_earlier_rows():
    B, Hq, Hkv, S, d = 1, 4, 1, 30, 16
    q, K, V = _gauss((B, Hq, S, d)), _gauss((B, Hkv, S, d)), _gauss((B, Hkv, S, d))
    a = prefill.causal_attention(q, K, V, [S])
    K2, V2 = K.copy(), V.copy()
    K2[:, :, 17:] = _gauss((B, Hkv, S - 17, d))
    V2[:, :, 17:] = _gauss((B, Hkv, S - 17, d))
    b = prefill.causal_attention(q, K2, V2, [S])
    np.testing.assert_array_equal(a[:, :, :17], b[:, :, :17])
    assert not np.allclose(a[:, :, 17:], b[:, :, 17:])


def test_last_row_equals_dense_decode_oracle():
    """The last prompt row attends every key: the C oracle's dense decode
    attention (its own GQA mapping, fp64 softmax) gives the same row."""
    B, Hq, Hkv, S, d = 2, 8, 2, 70, 128
    q, K, V = _gauss((B, Hq, S, d)), _gauss((B, Hkv, S, d)), _gauss((B, Hkv, S, d))
    L = np.array([70, 33], np.int32)
    out = prefill.causal_attention(q, K, V, L)
    q_last = np.stack([q[b, :, L[b] - 1] for b in range(B)])
    dense = oracle.dense_attention(q_last, K, V, L, 1.0 / np.sqrt(d))
    for b in range(B):
        np.testing.assert_allclose(out[b, :, L[b] - 1], dense[b], rtol=1e-5, atol=1e-6)
    # rows past the length are left zero
    assert not out[1, :, 33:].any()


def test_abs_weighted_values_bounds_output():
    B, Hq, Hkv, S, d = 1, 2, 1, 25, 16
    q, K, V = _gauss((B, Hq, S, d)), _gauss((B, Hkv, S, d)), _gauss((B, Hkv, S, d))
    out = prefill.causal_attention(q, K, V, [S])
    bound = prefill.abs_weighted_values(q, K, V, [S])
    assert (np.abs(out) <= bound + 1e-12).all()
    # equal to |out| where all values in a column share a sign
    Vp = synth.bf16_bits(np.abs(synth.bf16_to_f32(V)))
    np.testing.assert_allclose(prefill.causal_attention(q, K, Vp, [S]),
                               prefill.abs_weighted_values(q, K, V, [S]), rtol=1e-12)


def test_prefill_codes_are_the_encoded_keys():
    B, Hq, Hkv, S, d, r = 1, 4, 2, 20, 128, 128
    q, K, V = _gauss((B, Hq, S, d)), _gauss((B, Hkv, S, d)), _gauss((B, Hkv, S, d))
    W = RNG.standard_normal((Hkv, d, r)).astype(np.float32)
    _, codes = prefill.prefill(q, K, V, W, [13])
    for h in range(Hkv):
        np.testing.assert_array_equal(codes[0, h, :13], oracle.encode(K[0, h, :13], W[h]))
    assert not codes[0, :, 13:].any()


def test_attention_rows_match_full_prefill_rows():
    B, Hq, Hkv, S, d = 1, 2, 1, 50, 16
    q, K, V = _gauss((B, Hq, S, d)), _gauss((B, Hkv, S, d)), _gauss((B, Hkv, S, d))
    full = prefill.causal_attention(q, K, V, [S])
    pos = [0, 1, 17, 49]
    rows = prefill.attention_rows(q[0, 1, pos], pos, K[0, 0], V[0, 0])
    np.testing.assert_allclose(rows, full[0, 1, pos], rtol=1e-12, atol=1e-14)
