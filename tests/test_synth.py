"""The seeded input generators (shared by the HIP path and the oracle)."""
import numpy as np
import torch

from hash_top_sparse_amd import synth


def test_bf16_rounding_matches_torch_rne():
    """bf16_bits is round-to-nearest-even, as torch's float32 -> bfloat16 cast."""
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0,
                        np.array([0.0, -0.0, 1.0, -1.0, 1.00390625, 1.005859375, 3e38, -3e-39],
                                 np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.bf16_bits(x), want)
    np.testing.assert_array_equal(synth.bf16_to_f32(want),
                                  torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_exact_recipe_values_and_determinism():
    s = synth.small_shape(B=2, Hq=4, Hkv=1, N=64, dist="exact", seed_base=1000)
    a = synth.make_inputs(s)
    b = synth.make_inputs(s)
    for f in ("q", "K", "V", "W"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    v = synth.bf16_to_f32(a.K) * 8
    assert (v == np.rint(v)).all() and np.abs(v).max() <= 32
    assert set(np.unique(a.W)) <= {-1.0, 0.0, 1.0}


def test_gauss_recipe_outliers_and_needles():
    s = synth.small_shape(B=1, Hq=8, Hkv=2, N=2000, k=64, seed_base=2000, outliers=4, needles=16)
    inp = synth.make_inputs(s)
    K = synth.bf16_to_f32(inp.K[0, 0]).astype(np.float64)
    ch = inp.outlier_ch[0]
    mask = np.ones(2000, bool)
    mask[inp.needle_pos[0, 0]] = False
    std = K[mask].std(0)
    assert (std[ch] > 6).all() and np.median(np.delete(std, ch)) < 1.2
    q = synth.bf16_to_f32(inp.q[0]).astype(np.float64)
    for j, p in enumerate(inp.needle_pos[0, 0]):
        qg = q[j % 4]
        cos = K[p] @ qg / np.linalg.norm(K[p]) / np.linalg.norm(qg)
        assert cos > 0.75
