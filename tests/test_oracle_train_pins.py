"""Pins of the W_H training-step oracle (oracle/train.py) against what the
HATA notes page ("Key design: Learning-to-Hash modelling") and mathematics
fix: the loss against explicit Python loops, the gradient against central
finite differences of the loss, the labels against a pure-Python sort and
closed cases, and special cases of each term."""
from __future__ import annotations

import math

import numpy as np
import pytest

from hash_top_sparse_amd import synth
from oracle import train

RNG = np.random.default_rng(4242)


def _inputs(J=5, n=20, d=16, r=8, seed=1):
    rng = np.random.default_rng(seed)
    q = synth.bf16_bits(rng.standard_normal((J, d)).astype(np.float32))
    k = synth.bf16_bits(rng.standard_normal((n, d)).astype(np.float32))
    pos = np.sort(rng.choice(n, size=J, replace=False)).astype(np.int32)
    W = rng.standard_normal((d, r)) / math.sqrt(d)
    return q, k, pos, W


def _py_loss(q, k, pos, S, W, sigma, eps, eta, lam):
    """The three terms by explicit loops over plain Python floats."""
    Q, K = train.bf16_to_f64(q).tolist(), train.bf16_to_f64(k).tolist()
    d, r = len(W), len(W[0])

    def h(x):
        out = []
        for c in range(r):
            z = sum(x[i] * W[i][c] for i in range(d))
            out.append(2.0 / (1.0 + math.exp(-sigma * z)) - 1.0)
        return out

    Hk = [h(x) for x in K]
    sim = bal = 0.0
    for j, qj in enumerate(Q):
        hq = h(qj)
        csum = [0.0] * r
        for i in range(int(pos[j]) + 1):
            sim += S[j][i] * sum((hq[c] - Hk[i][c]) ** 2 for c in range(r))
            for c in range(r):
                csum[c] += Hk[i][c]
        bal += sum(v * v for v in csum)
    dec2 = 0.0
    for a in range(r):
        for b in range(r):
            v = sum(W[i][a] * W[i][b] for i in range(d)) - (1.0 if a == b else 0.0)
            dec2 += v * v
    return eps * sim + eta * bal + lam * math.sqrt(dec2)


def test_loss_matches_explicit_loops():
    q, k, pos, W = _inputs()
    S = train.labels(q, k, pos)
    got = train.loss(q, k, pos, S, W, 1.5, 0.7, 0.3, 0.9)
    want = _py_loss(q, k, pos, S.tolist(), W.tolist(), 1.5, 0.7, 0.3, 0.9)
    assert abs(got[0] - want) <= 1e-9 * abs(want)
    assert abs(sum(got[1:]) - got[0]) <= 1e-12 * abs(got[0])


@pytest.mark.parametrize("eps,eta,lam", [(1.0, 0.0, 0.0), (0.0, 1.0, 0.0), (0.0, 0.0, 1.0), (0.6, 0.25, 2.0)])
def test_gradient_matches_central_differences(eps, eta, lam):
    """Every entry of dL/dW against (L(W + hE) - L(W - hE)) / 2h: a dropped
    term, a wrong sign or a transposed operand fails here."""
    q, k, pos, W = _inputs(seed=2)
    S = train.labels(q, k, pos)
    sigma = 1.3
    g = train.grad(q, k, pos, S, W, sigma, eps, eta, lam)
    hstep = 1e-6
    num = np.zeros_like(W)
    for a in range(W.shape[0]):
        for b in range(W.shape[1]):
            E = np.zeros_like(W)
            E[a, b] = hstep
            num[a, b] = (train.loss(q, k, pos, S, W + E, sigma, eps, eta, lam)[0]
                         - train.loss(q, k, pos, S, W - E, sigma, eps, eta, lam)[0]) / (2 * hstep)
    np.testing.assert_allclose(g, num, rtol=1e-5, atol=1e-6 * np.abs(num).max())


def test_train_step_descends():
    q, k, pos, W = _inputs(J=6, n=30, seed=3)
    S = train.labels(q, k, pos)
    args = (1.0, 1.0, 0.05, 0.5)
    W1, terms, g = train.train_step(q, k, pos, S, W, *args, lr=1e-3)
    np.testing.assert_allclose(W1, W - 1e-3 * g)
    assert train.loss(q, k, pos, S, W1, *args)[0] < terms[0]


def test_labels_match_python_sort_and_linear_ramp():
    q, k, pos, _ = _inputs(J=6, n=57, d=16, seed=4)
    S = train.labels(q, k, pos)
    Q, K = train.bf16_to_f64(q).tolist(), train.bf16_to_f64(k).tolist()
    for j in range(6):
        p = int(pos[j])
        sc = [sum(a * b for a, b in zip(Q[j], K[i])) for i in range(p + 1)]
        order = sorted(range(p + 1), key=lambda i: (-sc[i], i))
        P = max(1, -(-(p + 1) // 10))
        want = [-1.0] * (p + 1)
        for rank, i in enumerate(order[:P]):
            want[i] = 20.0 if P == 1 else 20.0 - 19.0 * rank / (P - 1)
        np.testing.assert_allclose(S[j, :p + 1], want, rtol=0, atol=1e-12)
        assert (S[j, p + 1:] == 0).all()


def test_labels_special_cases():
    d = 16
    q = synth.bf16_bits(np.ones((3, d), np.float32))
    k = synth.bf16_bits(np.ones((25, d), np.float32))  # every score equal: ties to the lower index
    pos = np.array([0, 9, 24], np.int32)
    S = train.labels(q, k, pos)
    assert S[0, 0] == 20.0 and (S[0, 1:] == 0).all()                 # one key: one positive
    assert S[1, 0] == 20.0 and (S[1, 1:10] == -1).all()              # 10 keys: 1 positive
    np.testing.assert_allclose(S[2, :3], [20.0, 10.5, 1.0])          # 25 keys: 3 positives
    assert (S[2, 3:25] == -1).all()


def test_orthonormal_W_has_no_decorrelation_loss():
    q, k, pos, _ = _inputs(d=16, r=8, seed=5)
    Wo, _ = np.linalg.qr(RNG.standard_normal((16, 8)))
    S = train.labels(q, k, pos)
    t = train.loss(q, k, pos, S, Wo, 1.0, 0.0, 0.0, 1.0)
    assert t[3] < 1e-12
    # (the Frobenius norm is not differentiable at W^T W = I, so no gradient
    # is pinned there; away from it the finite-difference pin covers it)


def test_large_sigma_hash_tends_to_sign():
    """h = 2 Sigmoid(sigma x W) - 1 -> sign(x W) as sigma grows (the decode
    encode's sign of the projection)."""
    q, _, _, W = _inputs(seed=6)
    Q = train.bf16_to_f64(q)
    z = Q @ W
    h = train.hash_relaxed(Q, W, 1e4)
    far = np.abs(z) > 1e-2
    np.testing.assert_allclose(h[far], np.sign(z[far]), atol=1e-12)
