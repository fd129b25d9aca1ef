"""GPU parity of hata_prefill (causal prompt attention with the prompt keys'
codes written to the cache) against the fp64 prefill oracle, through the C
ABI on seeded synthetic inputs.

Attention bar (derived from the kernel's arithmetic): the scores, softmax
statistics and every accumulation are fp32, and the weights are rounded to
bf16 before the value product (relative error <= 2^-9 each), so per element
|gpu - ref| <= 1e-4 + 1e-3 |ref| + 2^-8 * sum_j p_j |v_j| (twice the rounding
bound).  The error against the decode path's attention bar
(2e-3 + 1e-3 |ref| per element) is logged: worst ratio and the number of
elements past it.  Codes: bit-exact on the exact recipe, the flip allowance (|p| <
1e-4) otherwise.  Rows past each sequence's length are left untouched."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from hash_top_sparse_amd import synth
from helpers import ATOL, RTOL, bf16_tensor, check_codes, codes_np, gather_pages, paginate
from oracle import prefill as oprefill

pytestmark = pytest.mark.gpu

PV_ROUND = 2.0 ** -8
SENT_OUT = 7.25
SENT_CODE = 0x5A5A5A5A5A5A5A5A


def _sent(r):
    """Sentinel code word for r-bit rows (one int32 word at r = 32)."""
    return SENT_CODE if r >= 64 else 0x5A5A5A5A


def _log(msg):
    print(msg, flush=True)


def _bar(ref, absw):
    return 1e-4 + 1e-3 * np.abs(ref) + PV_ROUND * absw


def _check_out(got, ref, absw, what):
    """The kernel-derived bar (asserted); against the decode path's attention
    bar 2e-3 + 1e-3 |ref| the worst ratio and the count of elements past it
    are returned for the log (the bf16 weights can exceed it where a few
    keys with large |v| carry most of the weight)."""
    err = np.abs(got - ref)
    bar = _bar(ref, absw)
    assert (err <= bar).all(), f"{what}: max err {err.max():.3e}, worst excess {(err - bar).max():.3e}"
    ratio = err / (ATOL + RTOL * np.abs(ref))
    return float(ratio.max()), int((ratio > 1).sum()), int(ratio.size)


def _inputs(B, Hq, Hkv, q_rows, cap, r, seed, exact=False):
    rng = np.random.default_rng(seed)
    if exact:  # multiples of 1/8 in [-4, 4], W in {-1, 0, 1}: every projection exact in fp32
        def draw(shape):
            return synth.bf16_bits(rng.integers(-32, 33, size=shape).astype(np.float32) / 8)
        W = rng.integers(-1, 2, size=(Hkv, 128, r)).astype(np.float32)
    else:
        def draw(shape):
            return synth.bf16_bits(rng.standard_normal(shape).astype(np.float32))
        W = (rng.standard_normal((Hkv, 128, r)) / np.sqrt(128.0)).astype(np.float32)
    q = draw((B, Hq, q_rows, 128))
    K = draw((B, Hkv, cap, 128))
    V = draw((B, Hkv, cap, 128))
    return q, K, V, W


def _run(hb, q, K, V, W, lens, max_len, scale):
    B, Hq, q_rows, d = q.shape
    _, Hkv, cap, _ = K.shape
    r = W.shape[2]
    out = torch.full((B, Hq, q_rows, d), SENT_OUT, dtype=torch.float32, device="cuda")
    codes = hb.new_codes(B, Hkv, cap, r=r, fill=_sent(r))
    hb.prefill(bf16_tensor(q), bf16_tensor(K), bf16_tensor(V), torch.from_numpy(W).cuda(), codes,
               torch.from_numpy(np.asarray(lens, np.int32)).cuda(), max_len, scale, out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), codes_np(codes)


CASES = [
    # B, Hq, Hkv, lens, q_rows, cap, r, exact
    (2, 8, 2, [300, 77], 310, 320, 128, False),      # G = 4, ragged tails
    (1, 2, 2, [700], 700, 704, 64, False),           # G = 1: own rows span two key tiles
    (1, 4, 2, [130], 136, 130, 256, False),          # G = 2
    (1, 8, 1, [333], 333, 400, 32, False),           # G = 8, 16 positions per workgroup
    (3, 4, 1, [1, 64, 65], 80, 80, 128, False),      # one token, exactly one tile, one past it
    (1, 8, 2, [200], 200, 200, 128, True),           # exact recipe: codes bit-exact
]


@pytest.mark.parametrize("case", CASES, ids=[f"G{c[1] // c[2]}-r{c[6]}-{'x' if c[7] else 'g'}-{c[3]}"
                                             for c in CASES])
def test_prefill_matches_oracle(hata_gpu, case):
    B, Hq, Hkv, lens, q_rows, cap, r, exact = case
    _log(f"prefill B={B} Hq={Hq} Hkv={Hkv} lens={lens} r={r} exact={exact}")
    q, K, V, W = _inputs(B, Hq, Hkv, q_rows, cap, r, seed=8800 + sum(lens) + r, exact=exact)
    scale = 1.0 / np.sqrt(128.0)
    out, codes = _run(hata_gpu, q, K, V, W, lens, max(lens), scale)
    ref = oprefill.causal_attention(q, K, V, lens, scale)
    absw = oprefill.abs_weighted_values(q, K, V, lens, scale)
    flips = 0
    worst, past, total = 0.0, 0, 0
    for b in range(B):
        n = lens[b]
        w_, p_, t_ = _check_out(out[b, :, :n], ref[b, :, :n], absw[b, :, :n], f"b={b}")
        worst, past, total = max(worst, w_), past + p_, total + t_
        assert (out[b, :, n:] == SENT_OUT).all()
        for h in range(Hkv):
            flips += check_codes(codes[b, h, :n], K[b, h, :n], W[h], exact)
            assert (codes[b, h, n:] == np.uint64(_sent(r))).all()
    _log(f"  flips {flips}; err / (2e-3 + 1e-3|ref|): worst {worst:.3g}, {past} of {total} past 1")


def test_prefill_respects_max_len(hata_gpu):
    """Sequences longer than max_len are processed up to max_len only."""
    q, K, V, W = _inputs(2, 4, 1, 96, 96, 128, seed=8900)
    scale = 0.1
    out, codes = _run(hata_gpu, q, K, V, W, [96, 40], 50, scale)
    ref = oprefill.causal_attention(q, K, V, [50, 40], scale)
    absw = oprefill.abs_weighted_values(q, K, V, [50, 40], scale)
    for b, n in ((0, 50), (1, 40)):
        assert (np.abs(out[b, :, :n] - ref[b, :, :n]) <= _bar(ref[b, :, :n], absw[b, :, :n])).all()
        assert (out[b, :, n:] == SENT_OUT).all()
        assert (codes[b, 0, n:] == np.uint64(SENT_CODE)).all()
        check_codes(codes[b, 0, :n], K[b, 0, :n], W[0], False)


def test_prefill_equals_separate_encode(hata_gpu):
    """The codes the prefill writes equal those of hata_encode_append on the
    same keys (the bulk matrix-core path), bit for bit, on Gaussian inputs
    (both form the same two-term products in the same order; 786,432
    projections, so a different rounding would show)."""
    B, Hq, Hkv, n = 1, 8, 2, 3072
    q, K, V, W = _inputs(B, Hq, Hkv, n, n, 128, seed=8950)
    _, codes = _run(hata_gpu, q, K, V, W, [n], n, 0.0883883)
    sep = torch.zeros((B, Hkv, n, 2), dtype=torch.int64, device="cuda")
    hata_gpu.encode_append(bf16_tensor(K), torch.from_numpy(W).cuda(), sep, n_new=n)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(codes, codes_np(sep))


@pytest.mark.slow
@pytest.mark.parametrize("Hq,Hkv,N", [(32, 8, 32768), (32, 32, 8192)], ids=["gqa4-32k", "mha-8k"])
def test_prefill_full_size_sampled(hata_gpu, Hq, Hkv, N):
    """Long prompts of a Llama-3.1-8B-shaped layer (32 query / 8 KV heads,
    32K tokens) and of an MHA layer (32 heads, 8K tokens; one query head per
    KV head, own rows spanning two key tiles), d = 128, r = 128, inputs drawn
    on the device; sampled rows of every head against the oracle, sampled
    code rows against the encode oracle."""
    B, r = 1, 128
    G = Hq // Hkv
    _log(f"prefill full size N={N}")
    g = torch.Generator(device="cuda")
    g.manual_seed(9900)
    q = torch.randn((B, Hq, N, 128), generator=g, device="cuda").to(torch.bfloat16)
    K = torch.randn((B, Hkv, N, 128), generator=g, device="cuda").to(torch.bfloat16)
    V = torch.randn((B, Hkv, N, 128), generator=g, device="cuda").to(torch.bfloat16)
    W = torch.randn((Hkv, 128, r), generator=g, device="cuda") / np.sqrt(128.0)
    out = torch.full((B, Hq, N, 128), SENT_OUT, dtype=torch.float32, device="cuda")
    codes = torch.zeros((B, Hkv, N, 2), dtype=torch.int64, device="cuda")
    seq = torch.tensor([N], dtype=torch.int32, device="cuda")
    scale = 1.0 / np.sqrt(128.0)
    hata_gpu.prefill(q, K, V, W, codes, seq, N, scale, out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9901)
    pos = np.unique(np.concatenate([[0, 1, 31, 32, 63, 64, 127, 128, N - 65, N - 64, N - 1],
                                    rng.integers(0, N, size=9)]))
    Kb = K.view(torch.int16).cpu().numpy().view(np.uint16)
    Vb = V.view(torch.int16).cpu().numpy().view(np.uint16)
    Wn = W.cpu().numpy()
    worst, past, total = 0.0, 0, 0
    for h in range(Hq):
        qrows = q[0, h, torch.from_numpy(pos).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
        ref, absw = oprefill.attention_rows(qrows, pos, Kb[0, h // G], Vb[0, h // G], scale, with_abs=True)
        got = out[0, h, torch.from_numpy(pos).cuda()].cpu().numpy()
        w_, p_, t_ = _check_out(got, ref, absw, f"head {h}")
        worst, past, total = max(worst, w_), past + p_, total + t_
    cn = codes_np(codes)
    rows = np.unique(np.concatenate([pos, rng.integers(0, N, size=200)]))
    flips = 0
    for h in range(Hkv):
        flips += check_codes(cn[0, h, rows], Kb[0, h, rows], Wn[h], False)
    _log(f"  sampled {len(pos)} rows x {Hq} heads, {len(rows)} code rows x {Hkv} heads, flips {flips}, "
         f"err / (2e-3 + 1e-3|ref|): worst {worst:.3g}, {past} of {total} past 1")


PAGED_CASES = [
    # page rows, G, r, lens, spare pages
    (16, 4, 128, [300, 77], 3),
    (64, 1, 64, [700], 1),
    (256, 8, 256, [333], 0),
    (32, 2, 128, [1, 130], 2),
]


@pytest.mark.parametrize("case", PAGED_CASES, ids=[f"P{c[0]}-G{c[1]}-r{c[2]}-{c[3]}" for c in PAGED_CASES])
def test_paged_prefill_equals_contiguous_bitwise(hata_gpu, case):
    """The prompt's K/V read from, and its codes written to, shuffled pages:
    the same kernel through the block table, so outputs and codes are
    bit-identical to the contiguous prefill; other pool rows untouched."""
    P, G, r, lens, spare = case
    B, Hkv = len(lens), (1 if G == 8 else 2)
    Hq, q_rows, cap = G * Hkv, max(lens) + 3, max(lens) + 5
    _log(f"paged prefill P={P} G={G} r={r} lens={lens}")
    q, K, V, W = _inputs(B, Hq, Hkv, q_rows, cap, r, seed=8700 + P + r)
    scale = 1.0 / np.sqrt(128.0)
    out_c, codes_c = _run(hata_gpu, q, K, V, W, lens, max(lens), scale)
    mp = (cap + P - 1) // P
    num_pages = B * mp + spare
    perm = np.random.default_rng(8701 + P).permutation(num_pages)[:B * mp].astype(np.int32)
    bt = torch.from_numpy(perm.reshape(B, mp)).cuda()
    Kp = paginate(bf16_tensor(K), P, bt, num_pages)
    Vp = paginate(bf16_tensor(V), P, bt, num_pages)
    Cp = paginate(hata_gpu.new_codes(B, Hkv, cap, r=r, fill=_sent(r)), P, bt, num_pages, fill=_sent(r))
    out = torch.full((B, Hq, q_rows, 128), SENT_OUT, dtype=torch.float32, device="cuda")
    hata_gpu.prefill_paged(bf16_tensor(q), Kp, Vp, torch.from_numpy(W).cuda(), Cp, bt,
                           torch.from_numpy(np.asarray(lens, np.int32)).cuda(), max(lens), scale, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), out_c)     # sentinels past each length included
    got = codes_np(gather_pages(Cp, bt, cap))
    np.testing.assert_array_equal(got, codes_c)
    # pages no sequence owns keep their contents
    used = set(perm.tolist())
    for pg in range(num_pages):
        if pg not in used:
            assert (codes_np(Cp[pg]) == np.uint64(_sent(r))).all()
