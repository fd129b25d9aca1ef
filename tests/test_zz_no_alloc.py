"""hata_decode_step_noalloc (the decode step for callers that cannot
allocate, with the library's static scratch as its workspace) against
hata_decode_step with a caller workspace: the same codes, kept indices and
outputs, bit for bit, on two calls in a row -- the second with a smaller
input (fewer sequences, fewer KV heads, a shorter cache) -- and again after
calls of other sizes have used the scratch.  Called through the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

from hash_top_sparse_amd import binding, synth
from helpers import Dev, assert_close, gpu_build_cache

pytestmark = pytest.mark.gpu


def _noalloc(d: Dev, codes, k, out, idx):
    L = binding.load()
    fn = L.hata_decode_step_noalloc
    P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    fn.argtypes = [P, P, P, P, P, I, I, I, I, I, I64, P, I64, I, F, P, P, P]
    fn.restype = I
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = fn(d.q.data_ptr(), d.K.data_ptr(), d.V.data_ptr(), d.W.data_ptr(), codes.data_ptr(), d.B, d.Hq,
            d.Hkv, 128, 128, d.cap, d.seq.data_ptr(), d.max_len, k, d.inp.scale, out.data_ptr(),
            idx.data_ptr() if idx is not None else None, stream)
    return rc


def _case(hata_gpu, B, Hq, Hkv, N, k, seed, lens=None):
    s = synth.Shape(f"na-{B}-{Hq}-{Hkv}-{N}-{k}", B=B, Hq=Hq, Hkv=Hkv, N=N, k=k, dist="gauss",
                    seed_base=seed, outliers=4, needles=4)
    inp = synth.make_inputs(s, seq_lens=None if lens is None else np.array(lens, np.int32))
    d = Dev(inp)
    print(f"noalloc case B{B} Hq{Hq} Hkv{Hkv} N{N} k{k}", flush=True)
    codes_a = gpu_build_cache(hata_gpu, d)
    for b in range(B):
        codes_a[b, :, int(inp.seq_lens[b]) - 1] = 0x55
    codes_b = codes_a.clone()
    ws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP, B, Hq, Hkv, d.max_len, k)
    out_a = torch.full((B, Hq, 128), np.nan, dtype=torch.float32, device="cuda")
    out_b = out_a.clone()
    idx_a = torch.full((B, Hkv, k), -9, dtype=torch.int32, device="cuda")
    idx_b = idx_a.clone()
    hata_gpu.decode_step(d.q, d.K, d.V, d.W, codes_a, d.seq, d.max_len, k, inp.scale, out_a, ws, idx_a)
    assert _noalloc(d, codes_b, k, out_b, idx_b) == 0, binding.last_error_message()
    torch.cuda.synchronize()
    assert hata_gpu.workspace_check(ws) == 0
    assert torch.equal(codes_a, codes_b)
    np.testing.assert_array_equal(idx_b.cpu().numpy(), idx_a.cpu().numpy())
    assert_close(out_b.cpu().numpy(), out_a.cpu().numpy())
    assert torch.equal(out_a, out_b)  # the same kernel on the same inputs


def test_noalloc_equals_workspace_call_twice(hata_gpu):
    # a 128K-shaped call (8 units, 32 workgroups each), then a smaller one
    _case(hata_gpu, 1, 32, 8, 65536, 512, 9500)
    _case(hata_gpu, 2, 8, 2, 3000, 64, 9501, lens=[3000, 1717])


def test_noalloc_after_other_sizes(hata_gpu):
    # MHA (one workgroup per unit), a single unit, then the large shape again:
    # every call clears the flags it uses, whatever the earlier calls left
    _case(hata_gpu, 8, 8, 8, 4096, 128, 9502)
    _case(hata_gpu, 1, 4, 1, 20000, 256, 9503)
    _case(hata_gpu, 1, 32, 8, 65536, 512, 9504)


def test_noalloc_rejects_sizes_beyond_the_scratch(hata_gpu):
    # 64 units of 64K tokens at G = 8, r = 128 need more than the static scratch
    L = binding.load()
    fn = L.hata_decode_step_noalloc
    P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    fn.argtypes = [P, P, P, P, P, I, I, I, I, I, I64, P, I64, I, F, P, P, P]
    fn.restype = I
    A = P(0x10000)
    rc = fn(A, A, A, A, A, 64, 512, 64, 128, 128, 65536, A, 65536, 512, 0.1, A, None, None)
    assert rc == 5  # HATA_ERR_WORKSPACE, before anything is launched
    assert "static scratch" in binding.last_error_message()
