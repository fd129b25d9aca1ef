"""Oracle for the W_H training step -- TEST INFRASTRUCTURE ONLY.

Only the test-suite and the benchmark's CPU leg may import this module; the
HIP library shares no code with it.  Everything is numpy in fp64.

Follows the HATA notes page, section "Key design", subsection
"Learning-to-Hash modelling":
  * hash  h(x) = 2 * Sigmoid(sigma * x W_H) - 1   (x a row vector, W_H [d, r]);
  * objective, the sum of three terms:
      similarity   eps * sum_j sum_i s_ji * ||h(q_j) - h(k_ji)||^2
      bit balance  eta * sum_j ||sum_i h(k_ji)||^2
      decorrelation lam * ||W_H^T W_H - I_r||
  * training pairs: for a sampled query q_j, its keys k_1..k_j (the causal
    prefix) are scored by q.k; the top 10% are positives with labels that
    fall linearly over [1, 20], the other 90% negatives with label -1.

Readings where the page is silent (listed in the design notes):
  * the norm of the decorrelation term is the Frobenius norm, not squared;
  * query j sits at position p_j and pairs with keys 0..p_j (its own key
    included); the positives are the ceil((p_j + 1) / 10) keys of highest q.k
    (ties to the lower index), labelled s_max for the best down to s_min for
    the last, linearly in rank (s_max alone when there is one);
  * the bit-balance sum for query j runs over the same keys 0..p_j;
  * eps, eta, lam, sigma are arguments (the page gives no values); the
    training step is one plain gradient step W <- W - lr * dL/dW.

Parity status: labels pinned by a pure-Python sort on small cases and by
exact-arithmetic inputs; the loss pinned by explicit Python loops; the
gradient pinned by central finite differences of the loss (none unpinned).
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def labels(q_bits, k_bits, q_pos, pos_permille: int = 100, s_max: float = 20.0,
           s_min: float = 1.0) -> np.ndarray:
    """Pair labels S [J, n]: row j covers keys 0..q_pos[j] (zero beyond).
    The number of positives is ceil((p + 1) * pos_permille / 1000), at least 1
    (10% = 100 per mille), in integer arithmetic."""
    Q, K = bf16_to_f64(q_bits), bf16_to_f64(k_bits)
    J, n = Q.shape[0], K.shape[0]
    S = np.zeros((J, n))
    for j in range(J):
        p = int(q_pos[j])
        sc = K[:p + 1] @ Q[j]
        order = np.lexsort((np.arange(p + 1), -sc))  # score descending, index ascending
        P = max(1, ((p + 1) * int(pos_permille) + 999) // 1000)
        lab = np.full(p + 1, -1.0)
        if P == 1:
            lab[order[0]] = s_max
        else:
            lab[order[:P]] = s_max - (s_max - s_min) * np.arange(P) / (P - 1)
        S[j, :p + 1] = lab
    return S


def hash_relaxed(X: np.ndarray, W: np.ndarray, sigma: float) -> np.ndarray:
    # 2 * Sigmoid(z) - 1 == tanh(z / 2) exactly; the tanh form cannot overflow
    return np.tanh(0.5 * sigma * (X @ W))


def loss(q_bits, k_bits, q_pos, S, W, sigma, eps, eta, lam):
    """(total, similarity, balance, decorrelation)."""
    Q, K = bf16_to_f64(q_bits), bf16_to_f64(k_bits)
    W = np.asarray(W, np.float64)
    Hq, Hk = hash_relaxed(Q, W, sigma), hash_relaxed(K, W, sigma)
    sim = bal = 0.0
    for j in range(Q.shape[0]):
        p = int(q_pos[j])
        diff = Hq[j][None, :] - Hk[:p + 1]
        sim += float(np.sum(S[j, :p + 1] * np.sum(diff * diff, axis=1)))
        c = Hk[:p + 1].sum(axis=0)
        bal += float(c @ c)
    A = W.T @ W - np.eye(W.shape[1])
    dec = float(np.sqrt(np.sum(A * A)))
    return eps * sim + eta * bal + lam * dec, eps * sim, eta * bal, lam * dec


def grad(q_bits, k_bits, q_pos, S, W, sigma, eps, eta, lam) -> np.ndarray:
    """dL/dW [d, r] by the chain rule through h (dh/dz = (1 - h^2)/2, z = sigma x W)."""
    Q, K = bf16_to_f64(q_bits), bf16_to_f64(k_bits)
    W = np.asarray(W, np.float64)
    J, n = Q.shape[0], K.shape[0]
    Hq, Hk = hash_relaxed(Q, W, sigma), hash_relaxed(K, W, sigma)
    M = (np.arange(n)[None, :] <= np.asarray(q_pos)[:, None]).astype(np.float64)  # [J, n]
    Sm = S * M
    dHq = 2.0 * eps * (Sm.sum(axis=1)[:, None] * Hq - Sm @ Hk)
    C = M @ Hk
    dHk = 2.0 * eps * (Sm.sum(axis=0)[:, None] * Hk - Sm.T @ Hq) + 2.0 * eta * (M.T @ C)
    dZq = dHq * (1.0 - Hq * Hq) / 2.0
    dZk = dHk * (1.0 - Hk * Hk) / 2.0
    dW = sigma * (Q.T @ dZq + K.T @ dZk)
    A = W.T @ W - np.eye(W.shape[1])
    na = np.sqrt(np.sum(A * A))
    if na > 0:
        dW += lam * 2.0 * (W @ A) / na
    return dW


def train_step(q_bits, k_bits, q_pos, S, W, sigma, eps, eta, lam, lr):
    """One gradient step; returns (new W, loss terms before the step, gradient)."""
    g = grad(q_bits, k_bits, q_pos, S, W, sigma, eps, eta, lam)
    terms = loss(q_bits, k_bits, q_pos, S, W, sigma, eps, eta, lam)
    return np.asarray(W, np.float64) - lr * g, terms, g
