"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test names what it pins and where the fact comes from.  The method is
the one described in the paper notes on "HATA: Trainable and Hardware-
Efficient Hash-Aware Top-k Attention ...", section "Key design" (hash
function h(x) = 2*Sigmoid(sigma*x*W_H) - 1; HashEncode = matmul + Sign +
BitPack; Hamming distance = bitcount(xor); GQA aggregation; top-k; sparse
attention) and section "Overall framework" (exact attention over the kept
KV pairs).  No page prints a worked numeric example, so the pins are closed
forms, exact-arithmetic cases, invariants, library routines and brute force.
"""
import math

import numpy as np
import pytest
import scipy.special

from hash_top_sparse_amd import synth

RNG = np.random.default_rng(12345)


def _bits_of(codes_row, r):
    """Unpack one code (r/64 uint64 words) into r bits, bit c = word c//64 bit c%64."""
    out = []
    for c in range(r):
        out.append((int(codes_row[c // 64]) >> (c % 64)) & 1)
    return np.array(out, np.int64)


def _pm1(codes_row, r):
    return 2 * _bits_of(codes_row, r) - 1


def _gauss_rows(n, d, rng=RNG):
    return synth.bf16_bits(rng.standard_normal((n, d), dtype=np.float32))


def _gauss_W(d, r, rng=RNG):
    return (rng.standard_normal((d, r), dtype=np.float32) / np.float32(np.sqrt(128))).astype(np.float32)


# ---------------------------------------------------------------- popcount

def test_popcount_matches_python_bin(oracle_mod):
    """Loop popcount == Python's own binary-string count (independent routine)."""
    vals = [0, 1, 2**63, 2**64 - 1, 0xAAAAAAAAAAAAAAAA, 0x8000000000000001]
    vals += [int(v) for v in RNG.integers(0, 2**63, size=200, dtype=np.int64)]
    vals += [int(v) | (1 << 63) for v in RNG.integers(0, 2**63, size=50, dtype=np.int64)]
    for v in vals:
        assert oracle_mod.popcount64(v) == bin(v).count("1")


# ---------------------------------------------------------------- encode

def test_encode_identity_gives_sign_bits_lsb_first(oracle_mod):
    """W_H = I: bit c is (x_c >= 0), stored as bit c%64 of word c//64.
    Pins the projection orientation, the sign rule (>= 0 -> 1) and the
    packing order; values are read straight off x."""
    d = r = 128
    x = _gauss_rows(16, d)
    x[3, :10] = 0x0000  # +0.0 -> bit 1
    x[4, :] = 0x8000    # -0.0 everywhere -> all bits 1
    codes = oracle_mod.encode(x, np.eye(d, dtype=np.float32))
    xf = synth.bf16_to_f32(x)
    for row in range(x.shape[0]):
        want = (xf[row] >= 0).astype(np.int64)
        np.testing.assert_array_equal(_bits_of(codes[row], r), want)
    assert all(int(w) == 2**64 - 1 for w in codes[4])


def test_encode_nan_projection_gives_bit_zero(oracle_mod):
    """A NaN projection compares false with >= 0, so its bit is 0."""
    d = r = 128
    x = _gauss_rows(2, d)
    x[1, 5] = 0x7FC0  # bf16 quiet NaN: every projection of row 1 is NaN
    codes = oracle_mod.encode(x, np.eye(d, dtype=np.float32))
    assert all(int(w) == 0 for w in codes[1])


def test_encode_negated_identity_is_complement_except_zeros(oracle_mod):
    """W_H = -I: bit c = (-x_c >= 0), the complement of W_H = I except where
    x_c == 0 (both give 1)."""
    d = r = 128
    x = _gauss_rows(8, d)
    x[:, ::7] = 0
    a = oracle_mod.encode(x, np.eye(d, dtype=np.float32))
    b = oracle_mod.encode(x, -np.eye(d, dtype=np.float32))
    xf = synth.bf16_to_f32(x)
    for row in range(8):
        ba, bb = _bits_of(a[row], r), _bits_of(b[row], r)
        zero = xf[row] == 0
        np.testing.assert_array_equal(ba[~zero], 1 - bb[~zero])
        assert (ba[zero] == 1).all() and (bb[zero] == 1).all()


def test_encode_column_permutation_permutes_bits(oracle_mod):
    d, r = 128, 128
    x = _gauss_rows(10, d)
    W = _gauss_W(d, r)
    perm = RNG.permutation(r)
    a = oracle_mod.encode(x, W)
    b = oracle_mod.encode(x, np.ascontiguousarray(W[:, perm]))
    for row in range(10):
        np.testing.assert_array_equal(_bits_of(b[row], r), _bits_of(a[row], r)[perm])


def test_encode_exact_inputs_match_integer_arithmetic(oracle_mod):
    """Exact recipe (x = a/8, W in {-1,0,1}): the projection is the integer
    sum_i a_i w_ic divided by 8, computed here in int64; codes and projections
    must equal it exactly, including the bits of exactly-zero projections."""
    shape = synth.small_shape(B=1, Hq=4, Hkv=1, N=64, dist="exact", seed_base=1000)
    inp = synth.make_inputs(shape)
    W = inp.W[0]
    x = inp.K[0, 0]
    codes, proj = oracle_mod.encode(x, W, return_proj=True)
    a = np.rint(synth.bf16_to_f32(x) * 8).astype(np.int64)
    Wi = W.astype(np.int64)
    P = a @ Wi  # int64, exact
    np.testing.assert_array_equal(proj.astype(np.float64) * 8, P.astype(np.float64))
    for row in range(x.shape[0]):
        np.testing.assert_array_equal(_bits_of(codes[row], 128), (P[row] >= 0).astype(np.int64))
    assert (P == 0).sum() > 0  # the zero-projection case is exercised


def test_encode_power_of_two_scaling_leaves_codes(oracle_mod):
    """h(2^m x) == h(x): the sign of the projection does not depend on a
    positive scale (the reason the sigmoid's sigma drops out at inference)."""
    d, r = 128, 128
    xf = RNG.standard_normal((20, d)).astype(np.float32)
    x = synth.bf16_bits(xf)
    W = _gauss_W(d, r)
    base = oracle_mod.encode(x, W)
    for m in (-3, 2, 5):
        xs = synth.bf16_bits(synth.bf16_to_f32(x) * np.float32(2.0**m))
        np.testing.assert_array_equal(oracle_mod.encode(xs, W), base)


def test_encode_projection_close_to_float64_matmul(oracle_mod):
    """fp32 projection vs numpy float64 matmul (x row-vector times W [d, r]):
    within the sequential-summation error bound, and identical bits wherever
    |p| exceeds that bound.  A transposed W or a dropped term fails."""
    d, r = 128, 128
    x = _gauss_rows(64, d)
    W = _gauss_W(d, r)
    codes, proj = oracle_mod.encode(x, W, return_proj=True)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    P = xf @ W.astype(np.float64)
    bound = d * 2.0**-23 * (np.abs(xf) @ np.abs(W.astype(np.float64)))
    assert (np.abs(proj - P) <= bound).all()
    for row in range(64):
        sure = np.abs(P[row]) > bound[row]
        np.testing.assert_array_equal(_bits_of(codes[row], r)[sure], (P[row][sure] >= 0).astype(np.int64))


def test_h_of_negated_input(oracle_mod):
    """Ham(h(x), h(-x)) = r - #{c : p_c == 0}: negating x flips every bit
    except those whose projection is exactly 0 (they stay 1)."""
    shape = synth.small_shape(N=200, dist="exact", seed_base=1000)
    inp = synth.make_inputs(shape)
    x = inp.K[0, 0]
    W = inp.W[0]
    neg = x ^ np.uint16(0x8000)
    a, pa = oracle_mod.encode(x, W, return_proj=True)
    b = oracle_mod.encode(neg, W)
    for row in range(x.shape[0]):
        ham = int(np.sum(_bits_of(a[row], 128) != _bits_of(b[row], 128)))
        assert ham == 128 - int(np.sum(pa[row] == 0))


def test_simhash_collision_rate(oracle_mod):
    """Random Gaussian W_H makes h a random-hyperplane (SimHash) code: the
    probability that a bit differs is theta/pi for inputs at angle theta
    (Charikar 2002; the random signed-projection LSH the HashAttention pages
    use as their baseline).  500 pairs x 128 bits at theta = pi/3."""
    d, r = 128, 128
    n = 500
    rng = np.random.default_rng(77)
    u = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    v -= (np.sum(u * v, 1) / np.sum(u * u, 1))[:, None] * u
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    v /= np.linalg.norm(v, axis=1, keepdims=True)
    theta = np.pi / 3
    y = np.cos(theta) * u + np.sin(theta) * v
    xb = synth.bf16_bits((u * 4).astype(np.float32))
    yb = synth.bf16_bits((y * 4).astype(np.float32))
    hams = []
    for i in range(n):
        W = _gauss_W(d, r, rng)
        cx = oracle_mod.encode(xb[i:i + 1], W)[0]
        cy = oracle_mod.encode(yb[i:i + 1], W)[0]
        hams.append(int(np.sum(_bits_of(cx, r) != _bits_of(cy, r))))
    rate = np.mean(hams) / r
    assert abs(rate - theta / np.pi) < 0.01, rate


# ---------------------------------------------------------------- Hamming

def test_hamming_equals_pm1_inner_product_identity(oracle_mod):
    """On +-1 codes a, b: Ham = (r - <a,b>)/2 and ||a-b||^2 = 4 Ham (ties the
    training loss's squared distance to the decode-time Hamming distance)."""
    r = 128
    words = RNG.integers(0, 2**63, size=(40, 2), dtype=np.int64).astype(np.uint64)
    words[:, 1] |= np.uint64(1 << 63)
    for i in range(39):
        S = oracle_mod.hamming_gqa(words[i:i + 1], words[i + 1:i + 2])[0]
        a, b = _pm1(words[i], r), _pm1(words[i + 1], r)
        assert 2 * S == r - int(a @ b)
        assert int(np.sum((a - b) ** 2)) == 4 * S


def test_hamming_metric_axioms(oracle_mod):
    codes = RNG.integers(0, 2**63, size=(30, 2), dtype=np.int64).astype(np.uint64)
    D = np.array([oracle_mod.hamming_gqa(codes[i:i + 1], codes) for i in range(30)])
    assert (np.diag(D) == 0).all()
    assert (D == D.T).all()
    assert ((D >= 0) & (D <= 128)).all()
    for i in range(30):
        assert (D[i][:, None] <= D[i][None, :] + D).all()  # D(i,j) <= D(i,k)+D(k,j)


def test_hamming_gqa_sum_matches_numpy_bitwise_count(oracle_mod):
    """Summed distance over G query codes == numpy's bitwise_count of the xor
    (library routine), per head and summed; G identical queries give G*Ham."""
    for G in (1, 2, 4, 8):
        q = RNG.integers(0, 2**63, size=(G, 2), dtype=np.int64).astype(np.uint64) ^ np.uint64(1 << 63)
        kc = RNG.integers(0, 2**63, size=(300, 2), dtype=np.int64).astype(np.uint64)
        S = oracle_mod.hamming_gqa(q, kc)
        want = np.zeros(300, np.int64)
        for g in range(G):
            want += np.bitwise_count(q[g][None, :] ^ kc).sum(1).astype(np.int64)
        np.testing.assert_array_equal(S, want)
        same = np.repeat(q[:1], G, axis=0)
        np.testing.assert_array_equal(oracle_mod.hamming_gqa(same, kc),
                                      G * oracle_mod.hamming_gqa(q[:1], kc))


# ---------------------------------------------------------------- top-k

def test_topk_matches_sorted_and_lexsort(oracle_mod):
    """First k of the (score, index) order, reported ascending; checked
    against Python's sorted and numpy's lexsort (library routines)."""
    for trial in range(200):
        n = int(RNG.integers(1, 60))
        k = int(RNG.integers(1, 70))
        S = RNG.integers(0, int(RNG.integers(1, 8)), size=n).astype(np.int32)  # many ties
        got = oracle_mod.topk(S, k)
        m = min(k, n)
        ref = sorted(sorted(range(n), key=lambda i: (S[i], i))[:m])
        assert list(got[:m]) == ref and (got[m:] == -1).all()
        lex = np.sort(np.lexsort((np.arange(n), S))[:m])
        np.testing.assert_array_equal(got[:m], lex)


def test_topk_special_cases(oracle_mod):
    S = np.full(50, 7, np.int32)
    np.testing.assert_array_equal(oracle_mod.topk(S, 10), np.arange(10))  # all equal
    got = oracle_mod.topk(np.arange(5, 0, -1).astype(np.int32), 8)        # k > n
    np.testing.assert_array_equal(got, [0, 1, 2, 3, 4, -1, -1, -1])
    S = RNG.integers(0, 513, size=4096).astype(np.int32)
    idx = oracle_mod.topk(S, 256)
    T = S[idx].max()
    assert np.sum(S < T) < 256 <= np.sum(S <= T)   # threshold invariant
    assert (np.diff(idx) > 0).all()


# ---------------------------------------------------------------- attention

def _attn_inputs(G=4, n=50, d=128, rng=RNG):
    q = _gauss_rows(G, d, rng)
    K = _gauss_rows(n, d, rng)
    V = _gauss_rows(n, d, rng)
    return q, K, V


def test_attention_single_row_returns_that_value_row(oracle_mod):
    q, K, V = _attn_inputs()
    out = oracle_mod.attention(q, K, V, np.array([17, -1, -1], np.int32), 1 / math.sqrt(128))
    for g in range(4):
        np.testing.assert_array_equal(out[g], synth.bf16_to_f32(V[17]))


def test_attention_equal_logits_give_mean(oracle_mod):
    q, K, V = _attn_inputs()
    q[:] = 0
    idx = np.array([1, 4, 9, 30], np.int32)
    out = oracle_mod.attention(q, K, V, idx, 0.1)
    mean = synth.bf16_to_f32(V[idx]).astype(np.float64).mean(0)
    for g in range(4):
        np.testing.assert_allclose(out[g], mean, rtol=1e-6, atol=1e-7)


def test_attention_all_rows_equals_scipy_softmax(oracle_mod):
    """Keeping every row (k = n) is dense attention; the dense form is built
    from scipy.special.softmax and a numpy matmul in float64."""
    q, K, V = _attn_inputs(n=200)
    scale = 1 / math.sqrt(128)
    out = oracle_mod.attention(q, K, V, np.arange(200, dtype=np.int32), scale)
    qf, Kf, Vf = (synth.bf16_to_f32(a).astype(np.float64) for a in (q, K, V))
    P = scipy.special.softmax(scale * qf @ Kf.T, axis=1)
    np.testing.assert_allclose(out, (P @ Vf).astype(np.float32), rtol=2e-6, atol=1e-7)


def test_attention_subset_equals_scipy_on_gathered_rows(oracle_mod):
    q, K, V = _attn_inputs(n=300)
    idx = np.sort(RNG.choice(300, 40, replace=False)).astype(np.int32)
    out = oracle_mod.attention(q, K, V, idx, 0.3)
    qf, Kf, Vf = (synth.bf16_to_f32(a).astype(np.float64) for a in (q, K[idx], V[idx]))
    P = scipy.special.softmax(0.3 * qf @ Kf.T, axis=1)
    np.testing.assert_allclose(out, (P @ Vf).astype(np.float32), rtol=2e-6, atol=1e-7)
    # order of idx does not matter; the output is a convex combination of V rows
    perm = RNG.permutation(idx)
    np.testing.assert_allclose(oracle_mod.attention(q, K, V, perm, 0.3), out, rtol=1e-6, atol=1e-7)
    lo, hi = Vf.min(0), Vf.max(0)
    assert ((out >= lo - 1e-6) & (out <= hi + 1e-6)).all()


# ---------------------------------------------------------------- whole step

@pytest.mark.parametrize("B,Hq,Hkv,N,k,d,r,dist", [
    (1, 4, 1, 40, 6, 16, 64, "gauss"),
    (2, 4, 2, 23, 30, 16, 64, "exact"),   # k > n
    (1, 2, 1, 33, 5, 128, 128, "gauss"),
    (1, 4, 1, 40, 6, 16, 32, "gauss"),    # 32-bit codes (one word, high half zero)
    (1, 2, 1, 21, 4, 16, 256, "gauss"),   # 256-bit codes
])
def test_decode_step_matches_pure_python_brute_force(oracle_mod, B, Hq, Hkv, N, k, d, r, dist):
    from oracle import brute

    shape = synth.Shape("brute", B=B, Hq=Hq, Hkv=Hkv, N=N, k=k, dist=dist, seed_base=9100, d=d, r=r)
    inp = synth.make_inputs(shape, seq_lens=np.array([N - 3 * b for b in range(B)], np.int32))
    if dist == "exact":
        # exact recipe draws W in {-1,0,1} at d = r = 128; re-draw it at this size
        inp.W = np.random.default_rng(5).integers(-1, 2, size=(Hkv, d, r)).astype(np.float32)
    else:
        inp.W = np.random.default_rng(5).standard_normal((Hkv, d, r)).astype(np.float32) / np.float32(np.sqrt(d))
    # the cache rows before the new token come from the pure-Python encoder
    words = (r + 63) // 64
    codes = np.zeros((B, Hkv, inp.cap, words), np.uint64)
    for b in range(B):
        for h in range(Hkv):
            for i in range(int(inp.seq_lens[b]) - 1):
                codes[b, h, i] = brute.encode(list(inp.K[b, h, i]), inp.W[h].tolist())
    res = oracle_mod.decode_step(inp.q, inp.K, inp.V, inp.W, codes, inp.seq_lens, k, inp.scale,
                                 want_scores=True)
    out_b, idx_b, codes_b, scores_b = brute.decode_step(
        inp.q.tolist(), inp.K.tolist(), inp.V.tolist(), inp.W.tolist(),
        codes.astype(object).tolist(), inp.seq_lens.tolist(), k, inp.scale)
    for b in range(B):
        n = int(inp.seq_lens[b])
        for h in range(Hkv):
            assert [int(v) for v in res["codes"][b, h, n - 1]] == [int(v) for v in codes_b[b][h][n - 1]]
            assert list(res["scores"][b, h, :n]) == scores_b[b][h]
            assert list(res["idx"][b, h]) == idx_b[b][h]
    np.testing.assert_allclose(res["out"], np.array(out_b, np.float64).astype(np.float32),
                               rtol=1e-6, atol=1e-7)


def test_decode_step_keep_all_equals_dense(oracle_mod):
    """k >= n: the kept set is every token, so the step's output equals dense
    attention over the whole cache."""
    shape = synth.small_shape(B=2, Hq=8, Hkv=2, N=120, k=200, seed_base=9200)
    inp = synth.make_inputs(shape)
    codes = oracle_mod.build_cache(inp.K, inp.W)
    res = oracle_mod.decode_step(inp.q, inp.K, inp.V, inp.W, codes, inp.seq_lens, inp.k, inp.scale)
    dense = oracle_mod.dense_attention(inp.q, inp.K, inp.V, inp.seq_lens, inp.scale)
    np.testing.assert_allclose(res["out"], dense, rtol=1e-6, atol=1e-7)
    assert (res["idx"][:, :, :120] == np.arange(120)).all() and (res["idx"][:, :, 120:] == -1).all()


def test_decode_step_appended_code_is_encode_of_new_key(oracle_mod):
    shape = synth.small_shape(B=2, Hq=8, Hkv=2, N=64, k=8, seed_base=9300)
    inp = synth.make_inputs(shape)
    codes = oracle_mod.build_cache(inp.K, inp.W)
    stale = codes.copy()
    stale[:, :, -1] = 0
    res = oracle_mod.decode_step(inp.q, inp.K, inp.V, inp.W, stale, inp.seq_lens, inp.k, inp.scale)
    np.testing.assert_array_equal(res["codes"], codes)


# ------------------------------------------- separate query and key encoders
# (HashAttention summary page, "Approach": independent query and key
# encoders.)  Pins: the shared case is the special case Wk = W, and with
# Wk = -W every key bit flips wherever the projection is nonzero (negating W
# negates every product and so the fp32 sum exactly), which turns each
# summed distance S into G*r - S.


def test_decode_step_key_encoder_equal_to_query_encoder_is_shared_case(oracle_mod):
    shape = synth.small_shape(B=2, Hq=8, Hkv=2, N=96, k=16, seed_base=9400)
    inp = synth.make_inputs(shape)
    codes = oracle_mod.build_cache(inp.K, inp.W)
    a = oracle_mod.decode_step(inp.q, inp.K, inp.V, inp.W, codes, inp.seq_lens, inp.k, inp.scale,
                               want_scores=True)
    b = oracle_mod.decode_step(inp.q, inp.K, inp.V, inp.W, codes, inp.seq_lens, inp.k, inp.scale,
                               want_scores=True, Wk=inp.W.copy())
    for key in ("out", "idx", "codes", "scores"):
        np.testing.assert_array_equal(a[key], b[key])


def test_decode_step_negated_key_encoder_complements_scores(oracle_mod):
    shape = synth.small_shape(B=2, Hq=8, Hkv=2, N=200, k=24, seed_base=9500)
    inp = synth.make_inputs(shape)
    G, r = 4, inp.W.shape[2]
    Wk = -inp.W
    shared = oracle_mod.decode_step(inp.q, inp.K, inp.V, inp.W, oracle_mod.build_cache(inp.K, inp.W),
                                    inp.seq_lens, inp.k, inp.scale, want_scores=True)
    sep = oracle_mod.decode_step(inp.q, inp.K, inp.V, inp.W, oracle_mod.build_cache(inp.K, Wk),
                                 inp.seq_lens, inp.k, inp.scale, want_scores=True, Wk=Wk)
    for b in range(2):
        n = int(inp.seq_lens[b])
        # Gaussian inputs: no projection is exactly zero, so the identity is exact
        np.testing.assert_array_equal(sep["scores"][b, :, :n], G * r - shared["scores"][b, :, :n])
        # the appended row is the key encoder's code of the new key
        np.testing.assert_array_equal(sep["codes"][b, :, n - 1],
                                      np.stack([oracle_mod.encode(inp.K[b, h, n - 1], Wk[h])
                                                for h in range(2)]))
        # so the kept set is the k tokens of LARGEST shared distance (ties to lower index)
        for h in range(2):
            s = shared["scores"][b, h, :n].astype(np.int64)
            order = np.lexsort((np.arange(n), -s))[: inp.k]
            assert list(sep["idx"][b, h]) == sorted(order.tolist())



# ------------------------------------------------ other code widths r
# (HATA notes list the code width among the method's knobs; the
# HashAttention summary page uses 32-bit signatures.)  Closed forms: with W
# the first r columns of the identity (r <= d) bit c is (x_c >= 0); with
# W = [I, -I] (r = 2d) bit c is (x_c >= 0) and bit d + c is (x_c <= 0).  The
# code of r bits occupies ceil(r/64) words with the bits past r zero.


@pytest.mark.parametrize("r", [32, 64, 256])
def test_encode_identity_columns_each_width(oracle_mod, r):
    d = 128
    x = synth.bf16_bits(RNG.standard_normal((40, d)).astype(np.float32))
    x[0, :8] = 0  # exact zeros: bit 1 in both halves of [I, -I]
    if r <= d:
        W = np.eye(d, dtype=np.float32)[:, :r]
    else:
        W = np.concatenate([np.eye(d, dtype=np.float32), -np.eye(d, dtype=np.float32)], axis=1)
    codes = oracle_mod.encode(x, W)
    assert codes.shape == (40, (r + 63) // 64)
    xf = synth.bf16_to_f32(x)
    for row in range(40):
        bits = _bits_of(codes[row], 64 * codes.shape[1])
        want = np.zeros(64 * codes.shape[1], np.int64)
        if r <= d:
            want[:r] = xf[row, :r] >= 0
        else:
            want[:d] = xf[row] >= 0
            want[d:2 * d] = xf[row] <= 0
        np.testing.assert_array_equal(bits, want)


@pytest.mark.parametrize("r", [32, 64, 256])
def test_hamming_each_width_counts_differing_bits(oracle_mod, r):
    d = 128
    x = synth.bf16_bits(RNG.standard_normal((30, d)).astype(np.float32))
    W = _gauss_W(d, r)
    c = oracle_mod.encode(x, W)
    q = c[:3]
    S = oracle_mod.hamming_gqa(q, c)
    for i in range(30):
        want = sum(int(np.sum(_bits_of(q[g], 64 * c.shape[1]) != _bits_of(c[i], 64 * c.shape[1])))
                   for g in range(3))
        assert S[i] == want
        assert 0 <= S[i] <= 3 * r
