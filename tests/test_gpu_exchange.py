"""The fused step's cross-workgroup exchange and its failure contract.

A unit's workgroups wait for each other twice per step (histogram windows,
then partial attention records), each wait bounded.  These tests force a wait
to give up from the host -- one workgroup's flag slot is set far behind the
others' epoch, so the flag the others wait for is never reached, and the
bound is set to a few thousand polls -- and check that the failure is
reported in the error word and in the outputs (NaN, kept indices -2) while
every other unit's results are unchanged and every kernel ends normally.

The forcing step writes the workspace directly and relies on its layout:
the error words occupy the first 256 bytes, then one 32-bit flag per
(unit, workgroup slot) with 64 slots per unit.
"""
import numpy as np
import pytest
import torch

from hash_top_sparse_amd import synth
from helpers import Dev, gpu_build_cache

pytestmark = pytest.mark.gpu

FLAGS_OFFSET = 256
SLOTS = 64


def _log(msg):
    print(msg, flush=True)


def _inputs(B, Hq, Hkv, N, k, seed):
    s = synth.Shape(f"x-{B}-{Hq}-{Hkv}-{N}-{k}", B=B, Hq=Hq, Hkv=Hkv, N=N, k=k, dist="gauss",
                    seed_base=seed, outliers=4, needles=0)
    return synth.make_inputs(s)


@pytest.mark.parametrize("B,Hq,Hkv,N,k", [(1, 32, 8, 32768, 512), (1, 4, 1, 8192, 256)])
def test_exchange_timeout_is_reported(hata_gpu, B, Hq, Hkv, N, k):
    inp = _inputs(B, Hq, Hkv, N, k, seed=9300 + Hkv)
    d = Dev(inp)
    _log(f"exchange timeout case B{B} Hq{Hq} Hkv{Hkv} N{N} k{k}")
    codes = gpu_build_cache(hata_gpu, d)
    ws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP, B, Hq, Hkv, d.max_len, k)
    out0 = torch.zeros((B, Hq, 128), dtype=torch.float32, device="cuda")
    idx0 = torch.zeros((B, Hkv, k), dtype=torch.int32, device="cuda")
    hata_gpu.decode_step(d.q, d.K, d.V, d.W, codes, d.seq, d.max_len, k, inp.scale, out0, ws, idx0)
    torch.cuda.synchronize()
    assert hata_gpu.workspace_check(ws) == 0

    # unit `bad`, workgroup slot 5: its flag far behind the epoch of the others
    bad = Hkv // 2
    flags = ws[FLAGS_OFFSET:FLAGS_OFFSET + 4 * SLOTS * B * Hkv].view(torch.int32)
    epoch = int(flags[bad * SLOTS].item())
    assert epoch > 0 and (flags[bad * SLOTS:(bad + 1) * SLOTS] == epoch).all()
    flags[bad * SLOTS + 5] = epoch - 1000
    hata_gpu.workspace_set_spin_limit(ws, 4000)
    out1 = torch.zeros_like(out0)
    idx1 = torch.zeros_like(idx0)
    hata_gpu.decode_step(d.q, d.K, d.V, d.W, codes, d.seq, d.max_len, k, inp.scale, out1, ws, idx1)
    torch.cuda.synchronize()
    assert hata_gpu.workspace_check(ws) & 1
    G = Hq // Hkv
    o1, i1 = out1.cpu().numpy(), idx1.cpu().numpy()
    # the failed unit is marked: most of its outputs NaN, kept indices -2
    assert np.isnan(o1[0, bad * G:(bad + 1) * G]).mean() > 0.5
    assert (i1[0, bad] == -2).sum() > 0
    # every other unit is exactly as before
    o0, i0 = out0.cpu().numpy(), idx0.cpu().numpy()
    for h in range(Hkv):
        if h != bad:
            np.testing.assert_array_equal(o1[0, h * G:(h + 1) * G], o0[0, h * G:(h + 1) * G])
            np.testing.assert_array_equal(i1[0, h], i0[0, h])

    # after a reset the workspace serves again, with the default bound
    hata_gpu.workspace_reset(ws)
    out2 = torch.zeros_like(out0)
    idx2 = torch.zeros_like(idx0)
    hata_gpu.decode_step(d.q, d.K, d.V, d.W, codes, d.seq, d.max_len, k, inp.scale, out2, ws, idx2)
    torch.cuda.synchronize()
    assert hata_gpu.workspace_check(ws) == 0
    np.testing.assert_array_equal(out2.cpu().numpy(), o0)
    np.testing.assert_array_equal(idx2.cpu().numpy(), i0)


def test_staged_step_without_idx_out(hata_gpu):
    """A shape whose step runs as separate kernels (more units times two
    workgroups than compute units, 33,000 tokens per unit) accepts idx_out =
    NULL: the kept list then lives in the workspace, and the output equals
    the call that asks for the indices, bit for bit."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    U = cus // 2 + 2
    N, k = 33000, 64
    _log(f"staged step without idx_out: {U} units x {N} tokens")
    g = torch.Generator(device="cuda").manual_seed(9411)
    q = torch.randn((1, U, 128), generator=g, device="cuda").to(torch.bfloat16)
    K = torch.randn((1, U, N, 128), generator=g, device="cuda").to(torch.bfloat16)
    V = torch.randn((1, U, N, 128), generator=g, device="cuda").to(torch.bfloat16)
    W = torch.randn((U, 128, 128), generator=g, device="cuda") * (1.0 / 128) ** 0.5
    seq = torch.tensor([N - 5], dtype=torch.int32, device="cuda")
    codes = torch.zeros((1, U, N, 2), dtype=torch.int64, device="cuda")
    hata_gpu.encode_append(K, W, codes, n_new=N)
    codes_b = codes.clone()
    ws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP, 1, U, U, N, k)
    assert ws.numel() >= U * N * 2  # the staged layout (a score of every token)
    out_a = torch.zeros((1, U, 128), dtype=torch.float32, device="cuda")
    out_b = torch.zeros_like(out_a)
    idx = torch.full((1, U, k), -9, dtype=torch.int32, device="cuda")
    hata_gpu.decode_step(q, K, V, W, codes, seq, N, k, 1.0 / 128 ** 0.5, out_a, ws, idx)
    hata_gpu.decode_step(q, K, V, W, codes_b, seq, N, k, 1.0 / 128 ** 0.5, out_b, ws, None)
    torch.cuda.synchronize()
    assert torch.equal(codes, codes_b)
    assert torch.equal(out_a, out_b)
    ix = idx.cpu().numpy()
    assert ((ix >= 0) & (ix < N - 5)).all()
    assert (np.diff(ix, axis=-1) > 0).all()


def test_fused_after_staged_on_one_workspace(hata_gpu):
    """One workspace, the same B and Hkv, three calls: a fused step (100
    units of 60,000 tokens: two workgroups per unit), a call whose longer
    context (70,000 tokens) runs the separate kernels, then the fused step
    again.  The separate kernels' buffers lie past the fused step's exchange
    area, so the third call reads the flags the first one left and equals it
    bit for bit."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    U = min(100, cus // 2 - 2)
    n_fused, n_staged, k = 60000, 70000, 64
    _log(f"fused after staged: {U} units, {n_fused} / {n_staged} tokens")
    g = torch.Generator(device="cuda").manual_seed(9420)
    q = torch.randn((1, U, 128), generator=g, device="cuda").to(torch.bfloat16)
    K = torch.randn((1, U, n_staged, 128), generator=g, device="cuda").to(torch.bfloat16)
    V = torch.randn((1, U, n_staged, 128), generator=g, device="cuda").to(torch.bfloat16)
    W = torch.randn((U, 128, 128), generator=g, device="cuda") * (1.0 / 128) ** 0.5
    codes = hata_gpu.new_codes(1, U, n_staged, r=128)
    hata_gpu.encode_append(K, W, codes, n_new=n_staged)
    ws_bytes = max(hata_gpu.workspace_bytes(hata_gpu.OP_DECODE_STEP, 1, U, U, n, k) for n in (n_fused, n_staged))
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    assert hata_gpu.workspace_bytes(hata_gpu.OP_DECODE_STEP, 1, U, U, n_staged, k) > \
        hata_gpu.workspace_bytes(hata_gpu.OP_DECODE_STEP, 1, U, U, n_fused, k)  # the staged layout
    scale = 1.0 / 128 ** 0.5
    seq_f = torch.tensor([n_fused], dtype=torch.int32, device="cuda")
    seq_s = torch.tensor([n_staged], dtype=torch.int32, device="cuda")
    outs, idxs = [], []
    for seq, n in ((seq_f, n_fused), (seq_s, n_staged), (seq_f, n_fused)):
        out = torch.zeros((1, U, 128), dtype=torch.float32, device="cuda")
        idx = torch.full((1, U, k), -9, dtype=torch.int32, device="cuda")
        hata_gpu.decode_step(q, K, V, W, codes, seq, n, k, scale, out, ws, idx)
        torch.cuda.synchronize()
        assert hata_gpu.workspace_check(ws) == 0
        outs.append(out.cpu().numpy())
        idxs.append(idx.cpu().numpy())
    np.testing.assert_array_equal(idxs[2], idxs[0])
    np.testing.assert_array_equal(outs[2], outs[0])
    assert (idxs[1] >= 0).all()
