"""GPU parity of hata_decode_step_paged: the cache rows of each sequence are
scattered over shuffled pages of K/V/code pools; the step must give the
oracle's results on the gathered contiguous cache (codes, kept set, output)
and agree with hata_decode_step on the contiguous cache."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from hash_top_sparse_amd import synth
from helpers import (Dev, assert_close, check_codes, codes_np, gather_pages as _gather, gpu_build_cache,
                     gpu_query_codes, oracle_units, paginate as _paginate)

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


CASES = [
    # B, Hq, Hkv, N, lens, k, P, r, dist, spare pages
    (2, 32, 8, 6000, [6000, 4321], 512, 16, 128, "gauss", 7),
    (3, 8, 8, 2100, [1, 700, 2049], 64, 256, 128, "exact", 0),
    (2, 8, 4, 3000, [3000, 1500], 100, 64, 64, "gauss", 3),
    (1, 16, 2, 1000, [999], 32, 128, 256, "gauss", 1),
    (2, 8, 1, 1500, [1500, 37], 16, 32, 32, "gauss", 2),
]


@pytest.mark.parametrize("case", CASES, ids=[f"P{c[6]}-r{c[7]}-G{c[1] // c[2]}-{c[8]}" for c in CASES])
def test_paged_step_matches_oracle_and_contiguous_step(hata_gpu, case):
    B, Hq, Hkv, N, lens, k, P, r, dist, spare = case
    _log(f"paged step B={B} Hq={Hq} Hkv={Hkv} lens={lens} k={k} P={P} r={r} {dist}")
    s = synth.Shape(f"paged-{B}-{Hq}-{Hkv}-{N}", B=B, Hq=Hq, Hkv=Hkv, N=N, k=k, r=r, dist=dist,
                    seed_base=7700 + P + r, outliers=4 if dist == "gauss" else 0,
                    needles=8 if dist == "gauss" else 0)
    inp = synth.make_inputs(s, seq_lens=np.array(lens, np.int32))
    d = Dev(inp)
    codes = gpu_build_cache(hata_gpu, d) if r == 128 else None
    if codes is None:
        codes = hata_gpu.new_codes(B, Hkv, d.cap, r=r)
        hata_gpu.encode_append(d.K, d.W, codes, n_new=d.cap)
    mp = (d.cap + P - 1) // P
    num_pages = B * mp + spare
    perm = np.random.default_rng(7701 + P).permutation(num_pages)[:B * mp].astype(np.int32)
    bt = torch.from_numpy(perm.reshape(B, mp)).cuda()
    Kp = _paginate(d.K, P, bt, num_pages)
    Vp = _paginate(d.V, P, bt, num_pages)
    Cp = _paginate(codes, P, bt, num_pages, fill=0x1234)
    Cp_before = Cp.clone()

    ws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP_PAGED, B, Hq, Hkv, d.max_len, k, r=r)
    out = torch.zeros((B, Hq, 128), dtype=torch.float32, device="cuda")
    idx = torch.zeros((B, Hkv, k), dtype=torch.int32, device="cuda")
    hata_gpu.decode_step_paged(d.q, Kp, Vp, d.W, Cp, bt, d.seq, d.max_len, k, inp.scale, out, ws, idx_out=idx)
    torch.cuda.synchronize()

    # only the appended rows changed in the pool
    got_codes = _gather(Cp, bt, d.cap)
    changed = (Cp != Cp_before).any(dim=-1)
    expect_changed = torch.zeros_like(changed)
    for b, n in enumerate(lens):
        pg = int(perm[b * mp + (n - 1) // P])
        expect_changed[pg, :, (n - 1) % P] = True
    assert not (changed & ~expect_changed).any()

    # oracle stages on the GPU's own codes (an allowed flip cannot cascade)
    cn = codes_np(got_codes)
    for b, n in enumerate(lens):
        for h in range(Hkv):
            check_codes(cn[b, h, n - 1:n], inp.K[b, h, n - 1:n], inp.W[h], dist == "exact")
    qc = gpu_query_codes(hata_gpu, d) if r == 128 else None
    if qc is None:
        qc4 = hata_gpu.new_codes(B, Hq, 1, r=r)
        hata_gpu.encode_append(d.q.view(B, Hq, 1, 128), d.W, qc4, n_new=1)
        qc = qc4.view(B, Hq, qc4.shape[-1])
    _, ridx, rout = oracle_units(inp, codes_np(qc), cn)
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    assert_close(out.cpu().numpy(), rout, "paged vs oracle")

    # the contiguous fused step on the same cache gives the same codes and kept set
    cws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP, B, Hq, Hkv, d.max_len, k, r=r)
    cout = torch.zeros_like(out)
    cidx = torch.zeros_like(idx)
    hata_gpu.decode_step(d.q, d.K, d.V, d.W, codes, d.seq, d.max_len, k, inp.scale, cout, cws, cidx)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        assert torch.equal(codes[b, :, :n], got_codes[b, :, :n])
    assert torch.equal(idx, cidx)
    assert_close(out.cpu().numpy(), cout.cpu().numpy(), "paged vs contiguous")


FUSED_CASES = [
    # B, Hq, Hkv, N, lens, k, P, spare pages
    (1, 32, 8, 20000, [20000], 512, 256, 5),      # several workgroups per unit (exchange path)
    (1, 32, 8, 20000, [20000], 512, 1024, 0),
    (2, 8, 8, 5000, [5000, 777], 64, 512, 2),      # G = 1
    (2, 64, 8, 3000, [3000, 1], 128, 256, 1),      # G = 8, a one-token sequence
    (1, 32, 8, 20000, [20000], 512, 16, 3),        # 16-row pages: page ids per lane
    (2, 8, 8, 5000, [5000, 777], 64, 32, 2),
    (2, 64, 8, 3000, [3000, 1], 128, 64, 1),
    # chunks of more than two ring batches, the appended row inside a middle
    # workgroup's chunk
    (2, 4, 1, 270000, [270000, 123457], 512, 256, 3),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[f"P{c[6]}-G{c[1] // c[2]}-N{c[3]}" for c in FUSED_CASES])
def test_fused_paged_step_equals_contiguous_step_bitwise(hata_gpu, case):
    """With 128-bit codes the paged step runs the fused kernel (one page id
    per 256-row batch for pages of >= 256 rows, per lane for smaller ones);
    it differs from the contiguous one only in its addresses, so codes, kept
    set and output must be bit-identical."""
    B, Hq, Hkv, N, lens, k, P, spare = case
    _log(f"fused paged B={B} Hq={Hq} Hkv={Hkv} lens={lens} k={k} P={P}")
    s = synth.Shape(f"fpaged-{B}-{Hq}-{Hkv}-{N}", B=B, Hq=Hq, Hkv=Hkv, N=N, k=k, dist="gauss",
                    seed_base=7900 + P, outliers=4, needles=8)
    inp = synth.make_inputs(s, seq_lens=np.array(lens, np.int32))
    d = Dev(inp)
    codes = gpu_build_cache(hata_gpu, d)
    mp = (d.cap + P - 1) // P
    num_pages = B * mp + spare
    perm = np.random.default_rng(7901 + P).permutation(num_pages)[:B * mp].astype(np.int32)
    bt = torch.from_numpy(perm.reshape(B, mp)).cuda()
    Kp = _paginate(d.K, P, bt, num_pages)
    Vp = _paginate(d.V, P, bt, num_pages)
    Cp = _paginate(codes, P, bt, num_pages, fill=0x1234)
    ws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP_PAGED, B, Hq, Hkv, d.max_len, k)
    out = torch.zeros((B, Hq, 128), dtype=torch.float32, device="cuda")
    idx = torch.zeros((B, Hkv, k), dtype=torch.int32, device="cuda")
    for rep in range(2):  # the workspace's flags carry over between calls
        hata_gpu.decode_step_paged(d.q, Kp, Vp, d.W, Cp, bt, d.seq, d.max_len, k, inp.scale, out, ws, idx_out=idx)
    cws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP, B, Hq, Hkv, d.max_len, k)
    cout = torch.zeros_like(out)
    cidx = torch.zeros_like(idx)
    hata_gpu.decode_step(d.q, d.K, d.V, d.W, codes, d.seq, d.max_len, k, inp.scale, cout, cws, cidx)
    torch.cuda.synchronize()
    assert hata_gpu.workspace_check(ws) == 0
    got_codes = _gather(Cp, bt, d.cap)
    for b, n in enumerate(lens):
        assert torch.equal(codes[b, :, :n], got_codes[b, :, :n])
    assert torch.equal(idx, cidx)
    assert torch.equal(out, cout)


@pytest.mark.slow
@pytest.mark.parametrize("P", [16, 256])
def test_fused_paged_step_full_size_bitwise(hata_gpu, P):
    """The 128K workload's shape (32 query / 8 KV heads, k = 512) over
    shuffled pages: bit-identical to the contiguous step."""
    B, Hq, Hkv, N, k = 1, 32, 8, 131072, 512
    _log(f"fused paged full size P={P}")
    g = torch.Generator(device="cuda")
    g.manual_seed(9700 + P)
    q = torch.randn((B, Hq, 128), generator=g, device="cuda").to(torch.bfloat16)
    K = torch.randn((B, Hkv, N, 128), generator=g, device="cuda").to(torch.bfloat16)
    V = torch.randn((B, Hkv, N, 128), generator=g, device="cuda").to(torch.bfloat16)
    W = torch.randn((Hkv, 128, 128), generator=g, device="cuda") / np.sqrt(128.0)
    codes = torch.zeros((B, Hkv, N, 2), dtype=torch.int64, device="cuda")
    hata_gpu.encode_append(K, W, codes, n_new=N)
    seq = torch.full((B,), N, dtype=torch.int32, device="cuda")
    mp = N // P
    bt = torch.randperm(B * mp + 3, generator=g, device="cuda")[:B * mp].to(torch.int32).view(B, mp)
    Kp, Vp = _paginate(K, P, bt, B * mp + 3), _paginate(V, P, bt, B * mp + 3)
    Cp = _paginate(codes, P, bt, B * mp + 3)
    ws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP_PAGED, B, Hq, Hkv, N, k)
    out = torch.zeros((B, Hq, 128), dtype=torch.float32, device="cuda")
    idx = torch.zeros((B, Hkv, k), dtype=torch.int32, device="cuda")
    hata_gpu.decode_step_paged(q, Kp, Vp, W, Cp, bt, seq, N, k, 0.0883883, out, ws, idx_out=idx)
    cws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP, B, Hq, Hkv, N, k)
    cout, cidx = torch.zeros_like(out), torch.zeros_like(idx)
    hata_gpu.decode_step(q, K, V, W, codes, seq, N, k, 0.0883883, cout, cws, cidx)
    torch.cuda.synchronize()
    assert hata_gpu.workspace_check(ws) == 0 and hata_gpu.workspace_check(cws) == 0
    assert torch.equal(idx, cidx)
    assert torch.equal(out, cout)
    assert torch.equal(_gather(Cp, bt, N), codes)


@pytest.mark.slow
def test_staged_paged_step_equals_fused_contiguous_step(hata_gpu):
    """A shape whose fused step fits on chip only without the paged step's
    page-id list (one unit of 8 query heads, 256-bit codes, k = 4096,
    1,114,112 cached rows: 17,408 per workgroup), so the paged step runs its
    separate kernels (row encode, Hamming scan, multi-workgroup top-k,
    gather attention) while the contiguous one is fused: kept sets and codes
    equal, outputs close."""
    B, Hq, Hkv, N, k, r, P = 1, 8, 1, 1114112, 4096, 256, 64
    _log(f"staged paged route N={N} r={r} k={k} P={P}")
    g = torch.Generator(device="cuda")
    g.manual_seed(9800)
    q = torch.randn((B, Hq, 128), generator=g, device="cuda").to(torch.bfloat16)
    K = torch.randn((B, Hkv, N, 128), generator=g, device="cuda").to(torch.bfloat16)
    V = torch.randn((B, Hkv, N, 128), generator=g, device="cuda").to(torch.bfloat16)
    W = torch.randn((Hkv, 128, r), generator=g, device="cuda") / np.sqrt(128.0)
    codes = torch.zeros((B, Hkv, N, r // 64), dtype=torch.int64, device="cuda")
    hata_gpu.encode_append(K, W, codes, n_new=N - 1)  # row N-1 is written by the steps
    seq = torch.full((B,), N, dtype=torch.int32, device="cuda")
    mp = N // P
    bt = torch.randperm(mp + 5, generator=g, device="cuda")[:mp].to(torch.int32).view(B, mp)
    Kp, Vp = _paginate(K, P, bt, mp + 5), _paginate(V, P, bt, mp + 5)
    Cp = _paginate(codes, P, bt, mp + 5)
    ws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP_PAGED, B, Hq, Hkv, N, k, r=r)
    out = torch.zeros((B, Hq, 128), dtype=torch.float32, device="cuda")
    idx = torch.zeros((B, Hkv, k), dtype=torch.int32, device="cuda")
    hata_gpu.decode_step_paged(q, Kp, Vp, W, Cp, bt, seq, N, k, 0.0883883, out, ws, idx_out=idx)
    cws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP, B, Hq, Hkv, N, k, r=r)
    cout, cidx = torch.zeros_like(out), torch.zeros_like(idx)
    hata_gpu.decode_step(q, K, V, W, codes, seq, N, k, 0.0883883, cout, cws, cidx)
    torch.cuda.synchronize()
    assert hata_gpu.workspace_check(ws) == 0 and hata_gpu.workspace_check(cws) == 0
    assert torch.equal(_gather(Cp, bt, N), codes)
    assert torch.equal(idx, cidx)
    assert_close(out.cpu().numpy(), cout.cpu().numpy().astype(np.float64), "staged paged vs fused contiguous")

    # and against the oracle, stage by stage on the device's own query codes
    _log("staged paged route vs oracle")
    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
    Kn, Vn, qn = bits(K[0, 0]), bits(V[0, 0]), bits(q[0])
    Wn = W[0].cpu().numpy()
    cn = codes_np(codes)[0, 0]
    check_codes(cn[N - 1:N], Kn[N - 1:N], Wn, False)
    qc = torch.zeros((B, Hq, 1, r // 64), dtype=torch.int64, device="cuda")
    hata_gpu.encode_append(q.view(B, Hq, 1, 128), W, qc, n_new=1)
    torch.cuda.synchronize()
    S = oracle.hamming_gqa(codes_np(qc)[0, :, 0], cn)
    ridx = oracle.topk(S, k)
    np.testing.assert_array_equal(idx.cpu().numpy()[0, 0], ridx)
    rout = oracle.attention(qn, Kn, Vn, ridx, 0.0883883)
    assert_close(out.cpu().numpy()[0], rout, "staged paged vs oracle")
