"""CPU pins of the fp32 error bounds used by the training-step GPU tests
(tests/train_bounds.py).  An independent fp32 evaluation of the same loss and
gradient (NumPy float32, its own summation orders) must stay inside both the
worst-case bounds and the probabilistic ones, for each loss term alone and
for all three together; the probabilistic bounds must be far below the size
of the values they bound; and an evaluation with a planted precision loss
(the relaxed hash rounded to bfloat16) must break them."""
import numpy as np
import pytest

from hash_top_sparse_amd import synth
from oracle import train
from train_bounds import grad_bound, grad_bound_prob, loss_bound, loss_bound_prob


def _bf16_round(x):
    b = np.ascontiguousarray(x, np.float32).view(np.uint32)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return b.view(np.float32)


def _f32_grad_and_loss(q_bits, k_bits, q_pos, S, W, sigma, eps, eta, lam, h_bf16=False):
    """fp32 evaluation of the gradient (the chain written with dense masks)
    and of the loss (from its expansion, as the device forms it)."""
    f = np.float32
    Q = train.bf16_to_f64(q_bits).astype(f)
    K = train.bf16_to_f64(k_bits).astype(f)
    W = W.astype(f)
    n, r = K.shape[0], W.shape[1]
    Hq = np.tanh(f(0.5 * sigma) * (Q @ W)).astype(f)
    Hk = np.tanh(f(0.5 * sigma) * (K @ W)).astype(f)
    if h_bf16:
        Hq, Hk = _bf16_round(Hq), _bf16_round(Hk)
    M = (np.arange(n)[None, :] <= np.asarray(q_pos)[:, None]).astype(f)
    Sm = (S * M).astype(f)
    rs, cs = Sm.sum(axis=1, dtype=f), Sm.sum(axis=0, dtype=f)
    P1 = Sm @ Hk
    dHq = f(2 * eps) * (rs[:, None] * Hq - P1)
    C = M @ Hk
    dHk = f(2 * eps) * (cs[:, None] * Hk - Sm.T @ Hq) + f(2 * eta) * (M.T @ C)
    dZq = dHq * (f(1) - Hq * Hq) / f(2)
    dZk = dHk * (f(1) - Hk * Hk) / f(2)
    g = f(sigma) * (Q.T @ dZq + K.T @ dZk)
    A = W.T @ W - np.eye(r, dtype=f)
    na = np.sqrt(np.sum(A * A, dtype=f))
    g = g + f(2 * lam) * (W @ A) / na
    sim = (np.sum(rs * np.sum(Hq * Hq, axis=1, dtype=f), dtype=f)
           - f(2) * np.sum(np.sum(Hq * P1, axis=1, dtype=f), dtype=f)
           + np.sum(cs * np.sum(Hk * Hk, axis=1, dtype=f), dtype=f))
    bal = np.sum(C * C, dtype=f)
    terms = np.array([f(eps) * sim, f(eta) * bal, f(lam) * na], np.float64)
    return g.astype(np.float64), np.array([terms.sum(), *terms])


def _case(J, n, r, seed):
    rng = np.random.default_rng(seed)
    q = synth.bf16_bits(rng.standard_normal((J, 128)).astype(np.float32))
    k = synth.bf16_bits(rng.standard_normal((n, 128)).astype(np.float32))
    pos = np.sort(rng.choice(n, size=J, replace=False)).astype(np.int32)
    W = (rng.standard_normal((128, r)) / np.sqrt(128.0)).astype(np.float32)
    S = train.labels(q, k, pos).astype(np.float32).astype(np.float64)
    return q, k, pos, S, W


TERMS = [(1e-3, 2e-4, 0.3), (1e-3, 0.0, 0.0), (0.0, 2e-4, 0.0), (0.0, 0.0, 0.3)]
TERM_IDS = ["all", "similarity", "balance", "decorrelation"]


@pytest.mark.parametrize("terms", TERMS, ids=TERM_IDS)
@pytest.mark.parametrize("J,n,r,seed", [(96, 1200, 64, 4040), (200, 800, 96, 4042)])
def test_fp32_evaluation_within_bounds(terms, J, n, r, seed):
    eps, eta, lam = (float(np.float32(t)) for t in terms)
    sigma = 1.5
    q, k, pos, S, W = _case(J, n, r, seed)
    g64 = train.grad(q, k, pos, S, W, sigma, eps, eta, lam)
    l64 = np.array(train.loss(q, k, pos, S, W, sigma, eps, eta, lam))
    g32, l32 = _f32_grad_and_loss(q, k, pos, S, W, sigma, eps, eta, lam)
    err, lerr = np.abs(g32 - g64), np.abs(l32 - l64)
    gmax = np.abs(g64).max()
    # worst case: valid, but far too loose to test anything
    assert (err <= grad_bound(q, k, pos, S, W, sigma, eps, eta, lam)).all()
    assert (lerr <= loss_bound(q, k, pos, S, W, sigma, eps, eta, lam)).all()
    # probabilistic: valid and tight
    gb = grad_bound_prob(q, k, pos, S, W, sigma, eps, eta, lam)
    lb = loss_bound_prob(q, k, pos, S, W, sigma, eps, eta, lam)
    assert (err <= gb).all(), f"max excess {(err - gb).max():.3e}"
    assert (lerr <= lb).all(), (lerr, lb)
    assert np.median(gb) < 2e-4 * gmax
    assert gb.max() < 1e-3 * gmax
    assert (lb <= 2e-4 * np.abs(l64) + 1e-30).all()


@pytest.mark.parametrize("terms", TERMS[:3], ids=TERM_IDS[:3])
def test_bf16_hash_breaks_the_bound(terms):
    """Rounding the relaxed hash to bfloat16 (a plausible precision slip in a
    kernel) must put some gradient elements outside the bound."""
    eps, eta, lam = (float(np.float32(t)) for t in terms)
    q, k, pos, S, W = _case(96, 1200, 64, 4040)
    g64 = train.grad(q, k, pos, S, W, 1.5, eps, eta, lam)
    gbad, _ = _f32_grad_and_loss(q, k, pos, S, W, 1.5, eps, eta, lam, h_bf16=True)
    gb = grad_bound_prob(q, k, pos, S, W, 1.5, eps, eta, lam)
    assert (np.abs(gbad - g64) > gb).mean() > 0.1
