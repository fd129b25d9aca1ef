"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (the library picks the same plan for the same shape).

Per workload: the code cache is built by the library's bulk encode and
checked against the oracle's encode on sampled rows (bit-exact on the exact
recipe, flip allowance otherwise); one fused decode step then runs and every
unit's kept index set must equal the oracle's (fed the GPU's codes), with the
attention output within tolerance.  The dense baseline is checked on sampled
units.  Workload 1 is checked exhaustively."""
import numpy as np
import pytest
import torch

import oracle
from hash_top_sparse_amd import synth
from helpers import Dev, assert_close, check_codes, codes_np, gpu_build_cache, gpu_query_codes, oracle_units

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [1, 2, 4, 3, 5])
def test_fullsize_workload(hata_gpu, cfg):
    shape = synth.CONFIGS[cfg]
    print(f"full-size workload {cfg}: {shape.name}", flush=True)
    inp = synth.make_inputs(shape)
    d = Dev(inp)
    exact = shape.dist == "exact"
    codes = gpu_build_cache(hata_gpu, d)
    torch.cuda.synchronize()
    cn = codes_np(codes)
    rng = np.random.default_rng(cfg)
    flips = 0
    for b in range(shape.B):
        for h in range(shape.Hkv):
            if exact:
                rows = np.arange(shape.N)
            else:
                rows = np.sort(rng.choice(shape.N, size=min(shape.N, 512 if shape.units > 16 else 2048),
                                          replace=False))
            flips += check_codes(cn[b, h, rows], inp.K[b, h, rows], inp.W[h], exact=exact)
    print(f"  cache sampled, allowed flips: {flips}", flush=True)
    # one fused step; row n-1 of the cache deliberately stale
    codes[:, :, shape.N - 1] = 0
    ws = hata_gpu.alloc_workspace(hata_gpu.OP_DECODE_STEP, shape.B, shape.Hq, shape.Hkv, shape.N, shape.k)
    out = torch.full((shape.B, shape.Hq, 128), np.nan, dtype=torch.float32, device="cuda")
    idx = torch.full((shape.B, shape.Hkv, shape.k), -9, dtype=torch.int32, device="cuda")
    hata_gpu.decode_step(d.q, d.K, d.V, d.W, codes, d.seq, d.max_len, shape.k, inp.scale, out, ws, idx)
    torch.cuda.synchronize()
    assert hata_gpu.workspace_check(ws) == 0
    cn = codes_np(codes)
    for b in range(shape.B):
        for h in range(shape.Hkv):
            check_codes(cn[b, h, shape.N - 1:], inp.K[b, h, shape.N - 1:], inp.W[h], exact=exact)
    qc = codes_np(gpu_query_codes(hata_gpu, d))
    _, ref_idx, ref_out = oracle_units(inp, qc, cn)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    err = assert_close(out.cpu().numpy(), ref_out)
    print(f"  step ok: max abs err {err[0]:.2e}, max rel err {err[1]:.2e}", flush=True)
    if shape.needles:
        # statistical stand-in for needle retrieval, not parity: with random
        # (untrained) W_H a needle at cosine 0.9 to one of the 4 group queries
        # scores about 210 +- 11 against a top-512 threshold near 229-233,
        # so most (not all) planted keys are kept
        got = idx.cpu().numpy()
        hit = tot = 0
        for b in range(shape.B):
            for h in range(shape.Hkv):
                pos = inp.needle_pos[b, h]
                pos = pos[pos >= 0]
                hit += np.isin(pos, got[b, h]).sum()
                tot += pos.size
        print(f"  needles kept: {hit}/{tot}", flush=True)
        assert hit >= 0.75 * tot
    # dense baseline on two sampled units
    dout = torch.zeros_like(out)
    dws = hata_gpu.alloc_workspace(hata_gpu.OP_DENSE_DECODE, shape.B, shape.Hq, shape.Hkv, shape.N, 1)
    hata_gpu.dense_decode(d.q, d.K, d.V, d.seq, d.max_len, inp.scale, dout, dws)
    got = dout.cpu().numpy()
    G = shape.G
    for (b, h) in [(0, 0), (shape.B - 1, shape.Hkv - 1)]:
        ref = oracle.attention(inp.q[b, h * G:(h + 1) * G], inp.K[b, h], inp.V[b, h],
                               np.arange(shape.N, dtype=np.int32), inp.scale)
        assert_close(got[b, h * G:(h + 1) * G], ref, "dense")
    print("  dense ok", flush=True)
