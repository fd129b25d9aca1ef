"""GPU parity: every stage of the HIP path against the CPU oracle, through the
C ABI.  Codes, scores and index sets bit-exact (encode judged exactly on the
exact recipe, within the sign-flip allowance on Gaussian inputs); attention
within |gpu - ref| <= 2e-3 + 1e-3 |ref| in fp32."""
import numpy as np
import pytest
import torch

import oracle
from hash_top_sparse_amd import synth
from helpers import (Dev, assert_close, check_codes, codes_np, codes_tensor, gpu_build_cache,
                     gpu_query_codes, oracle_units, scores_np)

pytestmark = pytest.mark.gpu


def _shape(B, Hq, Hkv, N, k, dist="gauss", seed=7000, needles=0):
    return synth.Shape(f"t-{B}-{Hq}-{Hkv}-{N}-{k}-{dist}", B=B, Hq=Hq, Hkv=Hkv, N=N, k=k, dist=dist,
                       seed_base=seed, outliers=4 if dist == "gauss" else 0, needles=needles)


def _log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ encode

@pytest.mark.parametrize("dist", ["exact", "gauss"])
def test_encode_queries_and_bulk_cache(hata_gpu, dist):
    s = _shape(2, 8, 2, 700, 32, dist=dist, seed=7100)
    inp = synth.make_inputs(s)
    d = Dev(inp)
    _log(f"encode {s.name}")
    qc = codes_np(gpu_query_codes(hata_gpu, d))
    cc = codes_np(gpu_build_cache(hata_gpu, d))
    G = s.G
    flips = 0
    for b in range(s.B):
        for h in range(s.Hkv):
            flips += check_codes(qc[b, h * G:(h + 1) * G], inp.q[b, h * G:(h + 1) * G], inp.W[h],
                                 exact=dist == "exact")
            flips += check_codes(cc[b, h], inp.K[b, h], inp.W[h], exact=dist == "exact")
    _log(f"allowed flips: {flips}")


def test_encode_append_writes_only_row_pos(hata_gpu):
    s = _shape(3, 4, 1, 200, 16, seed=7200)
    lens = np.array([200, 57, 1], np.int32)
    inp = synth.make_inputs(s, seq_lens=lens)
    d = Dev(inp)
    sentinel = np.full((3, 1, 200, 2), 0x5A5A5A5A5A5A5A5A, np.uint64)
    codes = codes_tensor(sentinel)
    pos = torch.from_numpy(lens - 1).cuda()
    hata_gpu.encode_append(d.K, d.W, codes, n_new=1, pos=pos)
    got = codes_np(codes)
    for b in range(3):
        n = int(lens[b])
        mask = np.ones(200, bool)
        mask[n - 1] = False
        assert (got[b, 0, mask] == sentinel[b, 0, mask]).all()
        check_codes(got[b, 0, n - 1:n], inp.K[b, 0, n - 1:n], inp.W[0], exact=False)


def test_encode_exact_identity_bit_order(hata_gpu):
    """W_H = I: bit c is the sign of input channel c (fixes the packing order)."""
    s = _shape(1, 4, 1, 64, 8, seed=7300)
    inp = synth.make_inputs(s)
    inp.W = np.eye(128, dtype=np.float32)[None]
    d = Dev(inp)
    cc = codes_np(gpu_build_cache(hata_gpu, d))
    xf = synth.bf16_to_f32(inp.K[0, 0])
    for i in range(64):
        bits = [(int(cc[0, 0, i, c // 64]) >> (c % 64)) & 1 for c in range(128)]
        assert bits == [int(v >= 0) for v in xf[i]]


# ------------------------------------------------------------------ Hamming + top-k

@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_hamming_scores_exact(hata_gpu, G):
    Hkv = 2
    s = _shape(2, G * Hkv, Hkv, 3000, 64, seed=7400 + G)
    lens = np.array([3000, 1234], np.int32)
    inp = synth.make_inputs(s, seq_lens=lens)
    d = Dev(inp)
    qc = gpu_query_codes(hata_gpu, d)
    cc = gpu_build_cache(hata_gpu, d)
    sc = torch.full((2, Hkv, 3000), -1, dtype=torch.int16, device="cuda")
    hata_gpu.hamming_scores(qc, cc, d.seq, d.max_len, sc)
    got = scores_np(sc)
    qn, cn = codes_np(qc), codes_np(cc)
    for b in range(2):
        n = int(lens[b])
        for h in range(Hkv):
            ref = oracle.hamming_gqa(qn[b, h * G:(h + 1) * G], cn[b, h, :n])
            np.testing.assert_array_equal(got[b, h, :n].astype(np.int32), ref)
            assert (got[b, h, n:] == 0xFFFF).all()   # rows past n untouched


TOPK_CASES = ["random", "ties", "all_equal", "k_ge_n", "n1", "max_score"]


@pytest.mark.parametrize("case", TOPK_CASES)
def test_topk_exact(hata_gpu, case):
    rng = np.random.default_rng(600 + TOPK_CASES.index(case))
    B, Hkv, cap = 2, 3, 5000
    k = 512
    lens = np.array([5000, 3333], np.int32)
    max_score = 512
    if case == "random":
        S = rng.integers(200, 320, size=(B, Hkv, cap))
    elif case == "ties":
        S = rng.integers(0, 4, size=(B, Hkv, cap))
    elif case == "all_equal":
        S = np.full((B, Hkv, cap), 77)
    elif case == "k_ge_n":
        k = 4096
        lens = np.array([300, 4096], np.int32)
        S = rng.integers(0, 513, size=(B, Hkv, cap))
    elif case == "n1":
        lens = np.array([1, 2], np.int32)
        S = rng.integers(0, 513, size=(B, Hkv, cap))
    else:
        max_score = 1024
        S = rng.choice([0, 1024, 1023], size=(B, Hkv, cap))
    sc = torch.from_numpy(S.astype(np.uint16).view(np.int16)).cuda()
    idx = torch.full((B, Hkv, k), -7, dtype=torch.int32, device="cuda")
    seq = torch.from_numpy(lens).cuda()
    hata_gpu.topk(sc, seq, int(lens.max()), k, max_score, idx)
    got = idx.cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            ref = oracle.topk(S[b, h, :lens[b]].astype(np.int32), k)
            np.testing.assert_array_equal(got[b, h], ref)


MULTI_TOPK_CASES = [
    # lens, k, score range (low, high), max_score
    ([20000, 4097], 512, (200, 330), 512),      # random; one length just past one chunk
    ([20000, 13000], 512, (0, 4), 512),          # heavy ties crossing chunk boundaries
    ([20000, 8192], 4096, (77, 78), 512),        # all equal: the first k rows
    ([20000, 100], 512, (0, 513), 512),          # a sequence shorter than k
    ([131072, 65536], 1, (0, 1025), 1024),       # k = 1, long rows
    ([40000, 40000], 2048, (0, 2049), 2048),     # widest bins (G r = 2048)
    ([20001, 9999], 512, (0, 8), 512),           # odd row stride: unaligned score rows read per score
]


@pytest.mark.parametrize("case", range(len(MULTI_TOPK_CASES)))
def test_topk_many_workgroups_exact(hata_gpu, case):
    """With its workspace, hata_topk splits long sequences over workgroups
    (chunk histograms, threshold, chunk counts, ordered compaction); the kept
    set must be the oracle's, including the lowest-index tie rule across
    chunks, and equal to the one-workgroup selection."""
    lens, k, (lo, hi), max_score = MULTI_TOPK_CASES[case]
    rng = np.random.default_rng(650 + case)
    B, Hkv, cap = 2, 2, max(lens)
    lens = np.array(lens, np.int32)
    S = rng.integers(lo, hi, size=(B, Hkv, cap))
    sc = torch.from_numpy(S.astype(np.uint16).view(np.int16)).cuda()
    seq = torch.from_numpy(lens).cuda()
    nbytes = hata_gpu.workspace_bytes(hata_gpu.OP_TOPK, B, Hkv * (max_score // 128), Hkv, cap, k)
    assert nbytes >= 4 * (B * Hkv * (max_score + 1) + 2 * B * Hkv * (1 + cap // 4096))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    idx = torch.full((B, Hkv, k), -7, dtype=torch.int32, device="cuda")
    hata_gpu.topk(sc, seq, cap, k, max_score, idx, ws=ws)
    one = torch.full_like(idx, -9)
    hata_gpu.topk(sc, seq, cap, k, max_score, one)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            ref = oracle.topk(S[b, h, :lens[b]].astype(np.int32), k)
            np.testing.assert_array_equal(got[b, h], ref)
    assert torch.equal(idx, one)


# ------------------------------------------------------------------ attention

@pytest.mark.parametrize("G", [1, 4, 8])
def test_sparse_decode_matches_oracle(hata_gpu, G):
    Hkv = 2
    s = _shape(2, G * Hkv, Hkv, 2000, 100, seed=7500 + G)
    inp = synth.make_inputs(s)
    d = Dev(inp)
    rng = np.random.default_rng(G)
    idx = np.full((2, Hkv, 100), -1, np.int32)
    for b in range(2):
        for h in range(Hkv):
            m = [100, 37, 1, 0][(b * Hkv + h) % 4]
            idx[b, h, :m] = np.sort(rng.choice(2000, m, replace=False))
    it = torch.from_numpy(idx).cuda()
    out = torch.full((2, G * Hkv, 128), np.nan, dtype=torch.float32, device="cuda")
    ws = hata_gpu.alloc_workspace(hata_gpu.OP_SPARSE_DECODE, 2, G * Hkv, Hkv, 100, 100)
    hata_gpu.sparse_decode(d.q, d.K, d.V, it, inp.scale, out, ws)
    got = out.cpu().numpy()
    for b in range(2):
        for h in range(Hkv):
            ref = oracle.attention(inp.q[b, h * G:(h + 1) * G], inp.K[b, h], inp.V[b, h], idx[b, h], inp.scale)
            if (idx[b, h] < 0).all():
                ref = np.zeros_like(ref)
            assert_close(got[b, h * G:(h + 1) * G], ref)


@pytest.mark.parametrize("G,N", [(4, 5000), (1, 777), (8, 300)])
def test_dense_decode_matches_oracle(hata_gpu, G, N):
    Hkv = 2
    s = _shape(2, G * Hkv, Hkv, N, 8, seed=7600 + G)
    lens = np.array([N, max(1, N // 3)], np.int32)
    inp = synth.make_inputs(s, seq_lens=lens)
    d = Dev(inp)
    out = torch.full((2, G * Hkv, 128), np.nan, dtype=torch.float32, device="cuda")
    ws = hata_gpu.alloc_workspace(hata_gpu.OP_DENSE_DECODE, 2, G * Hkv, Hkv, d.max_len, 1)
    hata_gpu.dense_decode(d.q, d.K, d.V, d.seq, d.max_len, inp.scale, out, ws)
    ref = oracle.dense_attention(inp.q, inp.K, inp.V, inp.seq_lens, inp.scale)
    assert_close(out.cpu().numpy(), ref)


# ------------------------------------------------------------------ fused step

STEP_CASES = [
    # B, Hq, Hkv, N, k, dist, lens
    (1, 4, 1, 4096, 256, "exact", None),          # exact recipe, many ties, Wg > 1
    (1, 32, 8, 8192, 512, "gauss", None),         # GQA-4, 8 units (XCD map)
    (3, 8, 2, 3000, 64, "gauss", [3000, 1500, 1]),  # ragged, n = 1
    (2, 8, 8, 700, 512, "gauss", [700, 300]),     # G = 1, k > n
    (1, 16, 2, 20000, 100, "gauss", None),        # G = 8
    (2, 4, 2, 1000, 5, "exact", [1000, 999]),     # G = 2, tiny k
    (8, 32, 32, 2048, 128, "gauss", None),        # 256 units, one workgroup each
    (1, 4, 4, 30000, 40, "gauss", None),          # G = 1 over many workgroups, most keep no row
    # workgroups keeping more than one attention batch (64 rows) of the
    # matrix-core path, for each G it serves
    (1, 8, 1, 4096, 1024, "exact", None),         # G = 8, many ties: up to 256 kept rows a workgroup
    (1, 2, 1, 4096, 1024, "exact", None),         # G = 2, the same
    (64, 32, 8, 1024, 300, "gauss", None),        # 512 units of one workgroup, G = 4: 300 kept rows each
    # chunks of more than two ring batches, the appended row inside a middle
    # workgroup's chunk (its key is encoded between the first two batches)
    (2, 4, 1, 270000, 512, "gauss", [270000, 123457]),
    # one query head per KV head, chunks of 9472 tokens: a full 32-token mask
    # word per thread and a partial one
    (1, 2, 2, 600000, 256, "gauss", None),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: f"B{c[0]}-Hq{c[1]}-Hkv{c[2]}-N{c[3]}-k{c[4]}-{c[5]}")
def test_decode_step_matches_oracle(hata_gpu, case):
    B, Hq, Hkv, N, k, dist, lens = case
    s = _shape(B, Hq, Hkv, N, k, dist=dist, seed=7700 + N % 97, needles=8 if dist == "gauss" else 0)
    lens = np.array(lens if lens else [N] * B, np.int32)
    inp = synth.make_inputs(s, seq_lens=lens)
    d = Dev(inp)
    _log(f"step case {case}")
    # cache rows [0, n-1) from the library's encode; row n-1 deliberately stale
    codes = gpu_build_cache(hata_gpu, d)
    for b in range(B):
        codes[b, :, int(lens[b]) - 1] = 0x1234
    ws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP, B, Hq, Hkv, d.max_len, k)
    out = torch.full((B, Hq, 128), np.nan, dtype=torch.float32, device="cuda")
    idx = torch.full((B, Hkv, k), -9, dtype=torch.int32, device="cuda")
    hata_gpu.decode_step(d.q, d.K, d.V, d.W, codes, d.seq, d.max_len, k, inp.scale, out, ws, idx)
    torch.cuda.synchronize()
    assert hata_gpu.workspace_check(ws) == 0
    cn = codes_np(codes)
    # appended code: same as the staged encode, and the oracle's within the allowance
    for b in range(B):
        n = int(lens[b])
        for h in range(Hkv):
            check_codes(cn[b, h, n - 1:n], inp.K[b, h, n - 1:n], inp.W[h], exact=dist == "exact")
    qc = codes_np(gpu_query_codes(hata_gpu, d))
    _, ref_idx, ref_out = oracle_units(inp, qc, cn)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    assert_close(out.cpu().numpy(), ref_out)


@pytest.mark.parametrize("G", [1, 4])
@pytest.mark.parametrize("pattern", ["clusters", "all-tied"])
def test_decode_step_concentrated_kept_rows(hata_gpu, G, pattern):
    """A unit of 64 workgroups of 512 tokens whose kept rows are concentrated
    in a few workgroups (some hold more than 256 tokens at or below the
    threshold, others none).  "clusters": 450 tokens of workgroup 0 and 200
    of workgroup 5 get codes within two bits of the bitwise majority of the
    unit's query codes (k = 512); "all-tied": every cached row has one code,
    so every score ties and the lowest-index rule decides (k = 300)."""
    N = 32768
    k = 512 if pattern == "clusters" else 300
    s = _shape(1, G, 1, N, k, seed=7950 + G)
    inp = synth.make_inputs(s)
    d = Dev(inp)
    _log(f"concentrated kept rows, G={G} {pattern}")
    qc = codes_np(gpu_query_codes(hata_gpu, d))[0]  # [G, 2] uint64
    rng = np.random.default_rng(7960 + G)
    cn = np.zeros((1, 1, N, 2), np.uint64)
    if pattern == "clusters":
        cn[0, 0] = rng.integers(0, 2 ** 64, size=(N, 2), dtype=np.uint64)
        bits = np.unpackbits(qc.view(np.uint8).reshape(G, 16), axis=1, bitorder="little").astype(np.int32)
        maj = (2 * bits.sum(axis=0) > G) | ((2 * bits.sum(axis=0) == G) & (bits[0] == 1))
        maj_words = np.packbits(maj.astype(np.uint8), bitorder="little").view(np.uint64)
        rows = np.r_[10:460, 5 * 512 + 20:5 * 512 + 220]
        for j in rows:
            c = maj_words.copy()
            for bpos in rng.choice(128, size=int(rng.integers(0, 3)), replace=False):
                c[bpos // 64] ^= np.uint64(1) << np.uint64(bpos % 64)
            cn[0, 0, j] = c
    else:
        cn[0, 0, :] = rng.integers(0, 2 ** 64, size=2, dtype=np.uint64)
    codes = codes_tensor(cn)
    ws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP, 1, G, 1, N, k)
    out = torch.full((1, G, 128), np.nan, dtype=torch.float32, device="cuda")
    idx = torch.full((1, 1, k), -9, dtype=torch.int32, device="cuda")
    hata_gpu.decode_step(d.q, d.K, d.V, d.W, codes, d.seq, N, k, inp.scale, out, ws, idx)
    torch.cuda.synchronize()
    assert hata_gpu.workspace_check(ws) == 0
    cg = codes_np(codes)
    np.testing.assert_array_equal(cg[0, 0, :N - 1], cn[0, 0, :N - 1])
    qc3 = qc.reshape(1, G, 2)
    scores, ref_idx, ref_out = oracle_units(inp, qc3, cg)
    S = scores[(0, 0)]
    T = int(np.sort(S, kind="stable")[k - 1])
    per_wg = np.bincount(np.arange(N) // 512, weights=(S <= T), minlength=64)
    _log(f"  T={T}, workgroups with more than 256 tokens at or below T: {int((per_wg > 256).sum())}, "
         f"with at most 256: {int((per_wg <= 256).sum())}")
    if pattern == "clusters":
        assert per_wg[0] > 256 and (per_wg <= 256).any()
    else:
        assert (per_wg > 256).all()
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    assert_close(out.cpu().numpy(), ref_out)


@pytest.mark.parametrize("B,Hq,Hkv,N,k", [(3, 32, 8, 4096, 256), (3, 4, 1, 3000, 64)])
def test_decode_step_invalid_lengths(hata_gpu, B, Hq, Hkv, N, k):
    """A sequence whose device-side length lies outside [1, cap] gets a zero
    output and an all -1 kept set, and its code rows stay untouched; the
    other sequences of the batch are unaffected (the units of such a sequence
    leave before any exchange)."""
    s = _shape(B, Hq, Hkv, N, k, seed=7950 + Hkv)
    inp = synth.make_inputs(s)
    d = Dev(inp)
    _log(f"invalid-length case B{B} Hq{Hq} Hkv{Hkv} N{N} k{k}")
    codes = gpu_build_cache(hata_gpu, d)
    before = codes_np(codes).copy()
    bad = {1: 0, 2: d.cap + 7}
    seq = d.seq.clone()
    for b, n in bad.items():
        seq[b] = n
    ws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP, B, Hq, Hkv, d.max_len, k)
    out = torch.full((B, Hq, 128), np.nan, dtype=torch.float32, device="cuda")
    idx = torch.full((B, Hkv, k), -9, dtype=torch.int32, device="cuda")
    hata_gpu.decode_step(d.q, d.K, d.V, d.W, codes, seq, d.max_len, k, inp.scale, out, ws, idx)
    torch.cuda.synchronize()
    assert hata_gpu.workspace_check(ws) == 0
    got_out, got_idx, cn = out.cpu().numpy(), idx.cpu().numpy(), codes_np(codes)
    G = Hq // Hkv
    for b in bad:
        assert (got_out[b] == 0).all()
        assert (got_idx[b] == -1).all()
        np.testing.assert_array_equal(cn[b], before[b])
    qc = codes_np(gpu_query_codes(hata_gpu, d))
    units = [(0, h) for h in range(Hkv)]
    _, ref_idx, ref_out = oracle_units(inp, qc, cn, units=units)
    np.testing.assert_array_equal(got_idx[0], ref_idx[0])
    assert_close(got_out[0], ref_out[0])
    assert G * Hkv == Hq


def test_decode_step_equals_staged_path(hata_gpu):
    B, Hq, Hkv, N, k = 2, 32, 8, 6000, 512
    s = _shape(B, Hq, Hkv, N, k, seed=7800, needles=16)
    inp = synth.make_inputs(s, seq_lens=np.array([6000, 4321], np.int32))
    d = Dev(inp)
    codes = gpu_build_cache(hata_gpu, d)
    staged_codes = codes.clone()
    ws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP, B, Hq, Hkv, d.max_len, k)
    out = torch.zeros((B, Hq, 128), dtype=torch.float32, device="cuda")
    idx = torch.zeros((B, Hkv, k), dtype=torch.int32, device="cuda")
    hata_gpu.decode_step(d.q, d.K, d.V, d.W, codes, d.seq, d.max_len, k, inp.scale, out, ws, idx)
    # staged: encode q, append k, Hamming, top-k, sparse attention
    qc = gpu_query_codes(hata_gpu, d)
    hata_gpu.encode_append(d.K, d.W, staged_codes, n_new=1, pos=(d.seq - 1).to(torch.int32))
    sc = torch.zeros((B, Hkv, N), dtype=torch.int16, device="cuda")
    hata_gpu.hamming_scores(qc, staged_codes, d.seq, d.max_len, sc)
    sidx = torch.zeros((B, Hkv, k), dtype=torch.int32, device="cuda")
    hata_gpu.topk(sc, d.seq, d.max_len, k, (Hq // Hkv) * 128, sidx)
    sout = torch.zeros_like(out)
    ws2 = hata_gpu.alloc_workspace(hata_gpu.OP_SPARSE_DECODE, B, Hq, Hkv, k, k)
    hata_gpu.sparse_decode(d.q, d.K, d.V, sidx, inp.scale, sout, ws2)
    torch.cuda.synchronize()
    assert torch.equal(codes, staged_codes)
    assert torch.equal(idx, sidx)
    assert_close(out.cpu().numpy(), sout.cpu().numpy(), "fused vs staged")


def test_decode_step_deterministic_and_workspace_reuse(hata_gpu):
    """Bitwise-identical reruns; one workspace reused across shapes whose plans
    use different numbers of workgroups per unit."""
    B, Hq, Hkv, k = 1, 32, 8, 512
    runs = []
    ws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP, B, Hq, Hkv, 65536, k)
    for N in (65536, 4096, 65536, 20000, 65536):
        s = _shape(B, Hq, Hkv, N, k, seed=7900)
        inp = synth.make_inputs(s)
        d = Dev(inp)
        need = hata_gpu.workspace_bytes(hata_gpu.OP_DECODE_STEP, B, Hq, Hkv, N, k)
        assert need <= ws.numel()
        codes = gpu_build_cache(hata_gpu, d)
        out = torch.zeros((B, Hq, 128), dtype=torch.float32, device="cuda")
        idx = torch.zeros((B, Hkv, k), dtype=torch.int32, device="cuda")
        hata_gpu.decode_step(d.q, d.K, d.V, d.W, codes, d.seq, d.max_len, k, inp.scale, out, ws, idx)
        torch.cuda.synchronize()
        assert hata_gpu.workspace_check(ws) == 0
        if N == 65536:
            runs.append((out.cpu().numpy().copy(), idx.cpu().numpy().copy(), codes_np(codes).copy()))
        else:
            qc = codes_np(gpu_query_codes(hata_gpu, d))
            _, ref_idx, ref_out = oracle_units(inp, qc, codes_np(codes))
            np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
            assert_close(out.cpu().numpy(), ref_out)
    for o, i, c in runs[1:]:
        assert np.array_equal(o.view(np.uint32), runs[0][0].view(np.uint32))
        assert np.array_equal(i, runs[0][1]) and np.array_equal(c, runs[0][2])


def test_stream_read_reads_every_word(hata_gpu):
    """The read-stream measurement kernel folds every 32-bit word of the
    buffer: the XOR of its 1024 workgroup words is the XOR of the buffer."""
    rng = np.random.default_rng(11)
    words = rng.integers(0, 2**32, size=(3 << 20) + 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros(1024, dtype=torch.int64, device="cuda")
    hata_gpu.stream_read(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().astype(np.uint64) & 0xFFFFFFFF)
    assert int(got) == int(np.bitwise_xor.reduce(words))


@pytest.mark.parametrize("dist", ["exact", "gauss"])
@pytest.mark.parametrize("n", [3000, 20000], ids=["4-tile-workgroups", "16-tile-workgroups"])
def test_bulk_encode_matches_row_encode(hata_gpu, dist, n):
    """The matrix-core bulk path and the per-row path agree: bit-identical on
    the exact recipe, within the flip allowance of each other otherwise.
    3000 rows run in workgroups of 4 tiles of 128 rows; 20000 rows in
    workgroups of 16 tiles, the last one ragged (every workgroup's last tile
    is written from all four waves' words)."""
    cap = n + 100
    s = _shape(2, 4, 2, n, 16, dist=dist, seed=7950 + n)
    inp = synth.make_inputs(s, cap=cap)
    d = Dev(inp)
    bulk = torch.zeros((2, 2, cap, 2), dtype=torch.int64, device="cuda")
    hata_gpu.encode_append(d.K, d.W, bulk, n_new=n)       # matrix cores
    rows = torch.zeros_like(bulk)
    step = 500 if n <= 3000 else 511                    # per-row path (below the bulk threshold)
    for start in range(0, n, step):
        pos = torch.full((2,), start, dtype=torch.int32, device="cuda")
        hata_gpu.encode_append(d.K, d.W, rows, n_new=min(step, n - start), pos=pos)
    torch.cuda.synchronize()
    a, b_ = codes_np(bulk), codes_np(rows)
    assert (a[:, :, n:] == 0).all()
    if dist == "exact":
        np.testing.assert_array_equal(a, b_)
    else:
        rng = np.random.default_rng(n)
        for b in range(2):
            for h in range(2):
                sel = np.sort(rng.choice(n, size=min(n, 3000), replace=False))
                check_codes(a[b, h, sel], inp.K[b, h, sel], inp.W[h], exact=False)
                check_codes(b_[b, h, sel], inp.K[b, h, sel], inp.W[h], exact=False)


# ------------------------------------- separate query and key encoders

QK_CASES = [
    # B, Hq, Hkv, N, k, dist, lens
    (1, 32, 8, 8192, 512, "gauss", None),         # GQA-4, the owner of row n-1 reloads W_Hk
    (8, 32, 32, 2048, 128, "gauss", None),        # one workgroup per unit: every workgroup owns its row
    (1, 4, 1, 4096, 256, "exact", None),          # exact recipe: codes bit-exact
    (2, 8, 2, 3000, 64, "gauss", [3000, 1]),      # ragged, n = 1 (the new key is the only token)
    # chunks of more than two ring batches: the key, inside a middle
    # workgroup's chunk, is projected with W_Hk between the first two batches
    (2, 4, 1, 270000, 256, "gauss", [270000, 200000]),
]


@pytest.mark.parametrize("case", QK_CASES, ids=lambda c: f"B{c[0]}-Hq{c[1]}-Hkv{c[2]}-N{c[3]}-k{c[4]}-{c[5]}")
def test_decode_step_qk_matches_oracle(hata_gpu, case):
    B, Hq, Hkv, N, k, dist, lens = case
    s = _shape(B, Hq, Hkv, N, k, dist=dist, seed=7900 + N % 89)
    lens = np.array(lens if lens else [N] * B, np.int32)
    inp = synth.make_inputs(s, seq_lens=lens)
    d = Dev(inp)
    _log(f"qk step case {case}")
    rng = np.random.default_rng(7950)
    if dist == "exact":
        Wk_np = rng.integers(-1, 2, size=inp.W.shape).astype(np.float32)
    else:
        Wk_np = (rng.standard_normal(inp.W.shape) / np.sqrt(128.0)).astype(np.float32)
    Wk = torch.from_numpy(Wk_np).cuda()
    # the cache holds key-encoder codes; row n-1 deliberately stale
    codes = torch.zeros((B, Hkv, d.cap, 2), dtype=torch.int64, device="cuda")
    hata_gpu.encode_append(d.K, Wk, codes, n_new=d.cap)
    for b in range(B):
        codes[b, :, int(lens[b]) - 1] = 0x1234
    ws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP, B, Hq, Hkv, d.max_len, k)
    out = torch.full((B, Hq, 128), np.nan, dtype=torch.float32, device="cuda")
    idx = torch.full((B, Hkv, k), -9, dtype=torch.int32, device="cuda")
    hata_gpu.decode_step_qk(d.q, d.K, d.V, d.W, Wk, codes, d.seq, d.max_len, k, inp.scale, out, ws, idx)
    torch.cuda.synchronize()
    assert hata_gpu.workspace_check(ws) == 0
    cn = codes_np(codes)
    for b in range(B):
        n = int(lens[b])
        for h in range(Hkv):  # the appended row is the key encoder's code
            check_codes(cn[b, h, n - 1:n], inp.K[b, h, n - 1:n], Wk_np[h], exact=dist == "exact")
    qc = codes_np(gpu_query_codes(hata_gpu, d))  # query codes from W_Hq
    _, ref_idx, ref_out = oracle_units(inp, qc, cn)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    assert_close(out.cpu().numpy(), ref_out)


@pytest.mark.parametrize("r", [128, 256])
def test_decode_step_qk_staged_shape(hata_gpu, r):
    """A shape whose per-unit chunk cannot stay on chip (130 units of 32,800
    tokens: two workgroups per unit would need 260 CUs) runs the separate
    kernels inside the call; the key row is still encoded with W_Hk.  Inputs
    drawn on the device; a sample of units is checked against the oracle."""
    B, Hq, Hkv, N, k = 1, 130, 130, 32800, 64
    g = torch.Generator(device="cuda")
    g.manual_seed(7990)
    q = torch.randn((B, Hq, 128), generator=g, device="cuda").to(torch.bfloat16)
    K = torch.randn((B, Hkv, N, 128), generator=g, device="cuda").to(torch.bfloat16)
    V = torch.randn((B, Hkv, N, 128), generator=g, device="cuda").to(torch.bfloat16)
    Wq = torch.randn((Hkv, 128, r), generator=g, device="cuda") / np.sqrt(128.0)
    Wk = torch.randn((Hkv, 128, r), generator=g, device="cuda") / np.sqrt(128.0)
    seq = torch.full((B,), N, dtype=torch.int32, device="cuda")
    codes = hata_gpu.new_codes(B, Hkv, N, r=r)
    wd = codes.shape[-1]
    hata_gpu.encode_append(K, Wk, codes, n_new=N)
    codes[:, :, N - 1] = 0x1234
    ws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP, B, Hq, Hkv, N, k, r=r)
    out = torch.zeros((B, Hq, 128), dtype=torch.float32, device="cuda")
    idx = torch.zeros((B, Hkv, k), dtype=torch.int32, device="cuda")
    _log(f"qk staged shape: 130 units x 32800, r={r}")
    hata_gpu.decode_step_qk(q, K, V, Wq, Wk, codes, seq, N, k, 1.0 / np.sqrt(128.0), out, ws, idx)
    torch.cuda.synchronize()
    qc = hata_gpu.new_codes(B, Hq, 1, r=r)
    hata_gpu.encode_append(q.view(B, Hq, 1, 128), Wq, qc, n_new=1)
    bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    qcn = codes_np(qc.view(B, Hq, wd))
    for h in (0, 1, 77, 129):
        kb, vb = bits(K[0, h]), bits(V[0, h])
        cn = codes_np(codes[0, h])
        check_codes(cn[N - 1:N], kb[N - 1:N], Wk[h].cpu().numpy(), exact=False)
        S = oracle.hamming_gqa(qcn[0, h:h + 1], cn)
        ix = oracle.topk(S, k)
        np.testing.assert_array_equal(idx[0, h].cpu().numpy(), ix)
        ref = oracle.attention(bits(q[0, h:h + 1]), kb, vb, ix, 1.0 / np.sqrt(128.0))
        assert_close(out[0, h:h + 1].cpu().numpy(), ref)


# ------------------------------------------------- other code widths r
# Codes of r in {32, 64, 256} bits (r/8 bytes per row: one int32 word at
# r = 32, r/64 int64 words otherwise): every stage against the oracle at that
# width.

def _wshape(B, Hq, Hkv, N, k, r, dist="gauss", seed=8100):
    return synth.Shape(f"w-{B}-{Hq}-{Hkv}-{N}-{k}-{r}-{dist}", B=B, Hq=Hq, Hkv=Hkv, N=N, k=k, dist=dist,
                       seed_base=seed, r=r, needles=8 if dist == "gauss" else 0)


def _wcache(hb, d: Dev, r: int) -> torch.Tensor:
    codes = hb.new_codes(d.B, d.Hkv, d.cap, r=r)
    hb.encode_append(d.K, d.W, codes, n_new=d.cap)
    return codes


def _wqcodes(hb, d: Dev, r: int) -> torch.Tensor:
    qc = hb.new_codes(d.B, d.Hq, 1, r=r)
    hb.encode_append(d.q.view(d.B, d.Hq, 1, 128), d.W, qc, n_new=1)
    return qc.view(d.B, d.Hq, qc.shape[-1])


@pytest.mark.parametrize("r", [32, 64, 256])
@pytest.mark.parametrize("dist", ["exact", "gauss"])
def test_encode_and_hamming_each_width(hata_gpu, r, dist):
    s = _wshape(2, 8, 2, 1500, 64, r, dist=dist, seed=8200 + r)
    inp = synth.make_inputs(s)
    d = Dev(inp)
    _log(f"width r={r} {dist}: encode + hamming")
    codes = _wcache(hata_gpu, d, r)
    cn = codes_np(codes)
    for b in range(2):
        for h in range(2):
            check_codes(cn[b, h], inp.K[b, h], inp.W[h], exact=dist == "exact")
    if r == 32:  # 4-byte rows: a row of another width would land in the next head's rows
        assert codes.dtype == torch.int32 and codes.shape[-1] == 1
    qc = _wqcodes(hata_gpu, d, r)
    sc = torch.zeros((2, 2, d.cap), dtype=torch.int16, device="cuda")
    hata_gpu.hamming_scores(qc, codes, d.seq, d.max_len, sc, r=r)
    torch.cuda.synchronize()
    qn, scn = codes_np(qc), sc.cpu().numpy().astype(np.int64)
    for b in range(2):
        n = int(inp.seq_lens[b])
        for h in range(2):
            np.testing.assert_array_equal(scn[b, h, :n], oracle.hamming_gqa(qn[b, h * 4:(h + 1) * 4], cn[b, h, :n]))


WIDTH_STEP_CASES = [
    # B, Hq, Hkv, N, k, dist
    (1, 32, 8, 8192, 512, "gauss"),      # GQA-4, 32 workgroups per unit
    (8, 32, 32, 2048, 128, "gauss"),     # one workgroup per unit
    (1, 16, 2, 20000, 100, "gauss"),     # G = 8
    (1, 4, 1, 4096, 256, "exact"),       # exact recipe, many ties
    (1, 4, 1, 270000, 256, "gauss"),     # chunks of more than two ring batches (key encoded between them)
]


@pytest.mark.parametrize("r", [32, 64, 256])
@pytest.mark.parametrize("case", WIDTH_STEP_CASES, ids=lambda c: f"B{c[0]}-Hq{c[1]}-Hkv{c[2]}-N{c[3]}-k{c[4]}-{c[5]}")
def test_decode_step_each_width(hata_gpu, case, r):
    B, Hq, Hkv, N, k, dist = case
    s = _wshape(B, Hq, Hkv, N, k, r, dist=dist, seed=8300 + N % 83)
    inp = synth.make_inputs(s)
    d = Dev(inp)
    _log(f"width r={r} step case {case}")
    codes = _wcache(hata_gpu, d, r)
    for b in range(B):
        codes[b, :, int(inp.seq_lens[b]) - 1] = 0x1234
    ws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP, B, Hq, Hkv, d.max_len, k, r=r)
    out = torch.full((B, Hq, 128), np.nan, dtype=torch.float32, device="cuda")
    idx = torch.full((B, Hkv, k), -9, dtype=torch.int32, device="cuda")
    hata_gpu.decode_step(d.q, d.K, d.V, d.W, codes, d.seq, d.max_len, k, inp.scale, out, ws, idx)
    torch.cuda.synchronize()
    assert hata_gpu.workspace_check(ws) == 0
    cn = codes_np(codes)
    for b in range(B):
        n = int(inp.seq_lens[b])
        for h in range(Hkv):
            check_codes(cn[b, h, n - 1:n], inp.K[b, h, n - 1:n], inp.W[h], exact=dist == "exact")
    qc = codes_np(_wqcodes(hata_gpu, d, r))
    _, ref_idx, ref_out = oracle_units(inp, qc, cn)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    assert_close(out.cpu().numpy(), ref_out)
