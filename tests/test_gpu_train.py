"""GPU parity of the hash-weight training step (hata_hash_labels,
hata_hash_train_step) against the fp64 oracle (oracle/train.py), through the
C ABI on seeded synthetic Q/K."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from hash_top_sparse_amd import synth
from helpers import bf16_tensor
from oracle import train

import train_bounds

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _qk(J, n, seed, exact=False):
    rng = np.random.default_rng(seed)
    if exact:  # multiples of 1/8 with |a| <= 8: every fp32 dot product is exact
        q = rng.integers(-8, 9, size=(J, 128)).astype(np.float32) / 8
        k = rng.integers(-8, 9, size=(n, 128)).astype(np.float32) / 8
    else:
        q = rng.standard_normal((J, 128)).astype(np.float32)
        k = rng.standard_normal((n, 128)).astype(np.float32)
    pos = np.sort(rng.choice(n, size=J, replace=False)).astype(np.int32)
    pos[0] = 0
    pos[-1] = n - 1
    return synth.bf16_bits(q), synth.bf16_bits(k), pos


@pytest.mark.parametrize("n", [1, 700, 3000, 8192])
def test_labels_exact_inputs_match_oracle(hata_gpu, n):
    J = min(24, n)
    q, k, pos = _qk(J, n, 9100 + n, exact=True)
    if n == 1:
        pos[:] = 0
    _log(f"labels exact n={n}")
    S = torch.full((J, n), np.nan, dtype=torch.float32, device="cuda")
    hata_gpu.hash_labels(bf16_tensor(q), bf16_tensor(k), torch.from_numpy(pos).cuda(), S)
    torch.cuda.synchronize()
    ref = train.labels(q, k, pos)
    got = S.cpu().numpy()
    np.testing.assert_array_equal(got > 0, ref > 0)      # the same positives
    np.testing.assert_array_equal(got == -1, ref == -1)  # the same negatives
    np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("n,pm,distinct", [(3000, 1, 0), (3000, 333, 0), (8192, 1000, 0), (2000, 100, 4),
                                            (5000, 250, 3)])
def test_labels_fractions_and_heavy_ties_match_oracle(hata_gpu, n, pm, distinct):
    """Other positive fractions (one per mille up to every key, where the
    ranking sorts all p + 1 keys) and key rows drawn from only a few distinct
    rows, so that nearly every query has a run of equal scores at its
    positive/negative boundary (ties go to the lower key index).  Exact
    inputs: every score is exact in fp32, so the labels must be equal."""
    J = 24
    q, k, pos = _qk(J, n, 9700 + n + pm, exact=True)
    if distinct:
        rng = np.random.default_rng(9701 + n)
        k = k[rng.integers(0, distinct, size=n)]
    _log(f"labels n={n} permille={pm} distinct={distinct}")
    S = torch.full((J, n), np.nan, dtype=torch.float32, device="cuda")
    hata_gpu.hash_labels(bf16_tensor(q), bf16_tensor(k), torch.from_numpy(pos).cuda(), S,
                         pos_permille=pm, s_max=7.5, s_min=0.5)
    torch.cuda.synchronize()
    ref = train.labels(q, k, pos, pos_permille=pm, s_max=7.5, s_min=0.5)
    got = S.cpu().numpy()
    np.testing.assert_array_equal(got > 0, ref > 0)
    np.testing.assert_array_equal(got == -1, ref == -1)
    np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-6)


def test_labels_gaussian_inputs_valid(hata_gpu):
    """fp32 scores may order near-ties differently from fp64: every
    disagreement must involve keys whose fp64 scores lie within 1e-4 of the
    positive/negative boundary, and each row keeps exactly P positives."""
    J, n = 32, 4096
    q, k, pos = _qk(J, n, 9200)
    S = torch.zeros((J, n), dtype=torch.float32, device="cuda")
    hata_gpu.hash_labels(bf16_tensor(q), bf16_tensor(k), torch.from_numpy(pos).cuda(), S)
    torch.cuda.synchronize()
    got = S.cpu().numpy()
    ref = train.labels(q, k, pos)
    Q, K = train.bf16_to_f64(q), train.bf16_to_f64(k)
    for j in range(J):
        p = int(pos[j])
        P = max(1, ((p + 1) * 100 + 999) // 1000)
        assert int((got[j, :p + 1] > 0).sum()) == P
        diff = np.nonzero((got[j, :p + 1] > 0) != (ref[j, :p + 1] > 0))[0]
        if diff.size:
            sc = K[:p + 1] @ Q[j]
            edge = np.sort(sc)[::-1][P - 1]
            assert np.all(np.abs(sc[diff] - edge) <= 1e-4 * max(1.0, abs(edge)))


@pytest.mark.parametrize("J,n,r", [(64, 1536, 64), (64, 1536, 128), (64, 1536, 256), (50, 1500, 128),
                                   (200, 3001, 96)])
def test_train_step_matches_oracle(hata_gpu, J, n, r):
    """Ragged shapes cover partial output tiles, a short last k split and
    the split-k partial sums (products over n with few output tiles)."""
    q, k, pos = _qk(J, n, 9300 + r + J + n)
    _check_step(hata_gpu, q, k, pos, r, 9400 + r + J + n)


@pytest.mark.parametrize("terms", [(1e-3, 2e-4, 0.3), (1e-3, 0.0, 0.0), (0.0, 2e-4, 0.0), (0.0, 0.0, 0.3)],
                         ids=["all", "similarity", "balance", "decorrelation"])
def test_train_step_full_size_per_term(hata_gpu, terms):
    """The training workload's full shape (512 sampled queries over 8192
    keys, 128 hash bits), with all three loss terms and with each term alone
    (the others' weights zero), so that an error in one term's gradient
    cannot hide under another's."""
    J, n, r = 512, 8192, 128
    q, k, pos = _qk(J, n, 9800)
    _check_step(hata_gpu, q, k, pos, r, 9801, terms=terms)


def test_train_step_unsorted_clustered_positions(hata_gpu):
    """Query positions need not be sorted or distinct: 300 queries (two
    batches of the mask-sum kernels) with runs of equal positions at both
    sides of 64-row chunk boundaries, the first and last key, and a cluster
    inside one chunk, in shuffled order."""
    J, n, r = 300, 1000, 128
    q, k, _ = _qk(J, n, 9600)
    rng = np.random.default_rng(9601)
    pos = np.concatenate([np.full(40, 63), np.full(30, 64), np.full(10, 0), np.full(10, n - 1),
                          rng.integers(128, 192, size=60), rng.integers(0, n, size=J - 150)]).astype(np.int32)
    pos = pos[rng.permutation(J)]
    _check_step(hata_gpu, q, k, pos, r, 9602)


def _check_step(hata_gpu, q, k, pos, r, seed, terms=(1e-3, 2e-4, 0.3)):
    """One device step against the fp64 oracle.  The gradient and the loss
    terms must lie within the per-element fp32 error bounds of
    tests/train_bounds.py (first-order probabilistic rounding analysis of
    the same evaluation); the hyper-parameters are fp32 values, so that both
    sides use the same ones."""
    J, n = q.shape[0], k.shape[0]
    rng = np.random.default_rng(seed)
    W0 = (rng.standard_normal((128, r)) / np.sqrt(128.0)).astype(np.float32)
    S = train.labels(q, k, pos).astype(np.float32).astype(np.float64)
    sigma, lr = 1.5, float(np.float32(0.02))
    eps, eta, lam = (float(np.float32(t)) for t in terms)
    _log(f"train step J={J} n={n} r={r} eps={eps:g} eta={eta:g} lam={lam:g}")
    W = torch.from_numpy(W0.copy()).cuda()
    grad = torch.zeros_like(W)
    loss = torch.zeros(4, dtype=torch.float32, device="cuda")
    ws = hata_gpu.hash_train_workspace(J, n, r)
    hata_gpu.hash_train_step(bf16_tensor(q), bf16_tensor(k), torch.from_numpy(pos).cuda(),
                             torch.from_numpy(S.astype(np.float32)).cuda(), W, sigma, eps, eta, lam, lr,
                             loss, ws, grad=grad)
    torch.cuda.synchronize()
    ref_g = train.grad(q, k, pos, S, W0, sigma, eps, eta, lam)
    ref_l = np.array(train.loss(q, k, pos, S, W0, sigma, eps, eta, lam))
    g = grad.cpu().numpy().astype(np.float64)
    gb = train_bounds.grad_bound_prob(q, k, pos, S, W0, sigma, eps, eta, lam)
    lb = train_bounds.loss_bound_prob(q, k, pos, S, W0, sigma, eps, eta, lam)
    err = np.abs(g - ref_g)
    _log(f"  max |err| / bound {float((err / gb).max()):.3g}, max bound / max |g| "
         f"{float(gb.max() / np.abs(ref_g).max()):.2e}")
    assert (err <= gb).all(), f"{int((err > gb).sum())} elements outside, worst {(err / gb).max():.3g}x"
    lerr = np.abs(loss.cpu().numpy().astype(np.float64) - ref_l)
    assert (lerr <= lb).all(), (lerr, lb)
    # the device forms W - lr * g, lr as fp32, with one fused multiply-add:
    # one fp32 rounding of the updated value, at most half an ulp of it
    # (2^-24 relative); the bound is set at twice that
    np.testing.assert_allclose(W.cpu().numpy(), W0.astype(np.float64) - lr * g,
                               rtol=2.0 ** -23, atol=1e-30)


def test_train_steps_descend_on_device(hata_gpu):
    J, n, r = 128, 2048, 128
    q, k, pos = _qk(J, n, 9500)
    qd, kd, pd = bf16_tensor(q), bf16_tensor(k), torch.from_numpy(pos).cuda()
    S = torch.zeros((J, n), dtype=torch.float32, device="cuda")
    hata_gpu.hash_labels(qd, kd, pd, S)
    W = (torch.randn((128, r), generator=torch.Generator().manual_seed(3)) / np.sqrt(128.0)).cuda()
    loss = torch.zeros(4, dtype=torch.float32, device="cuda")
    ws = hata_gpu.hash_train_workspace(J, n, r)
    seen = []
    for _ in range(8):
        hata_gpu.hash_train_step(qd, kd, pd, S, W, 1.0, 1e-3, 1e-4, 0.1, 0.01, loss, ws)
        seen.append(float(loss[0].item()))
    assert seen[-1] < seen[0]
