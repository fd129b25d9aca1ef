"""Per-element error bounds for an fp32 evaluation of the hash-weight training
step's loss and gradient (test logic; the oracle computes the values).

The gradient follows the chain the oracle writes out (oracle/train.py):
Z = sigma X W, H = tanh(Z/2), the label-weighted sums, dH, dZ = dH (1 - H^2)/2
and dW = sigma (Q^T dZq + K^T dZk) + 2 lam W A / ||A||_F with A = W^T W - I.
Every quantity computed in fp32 carries an absolute error bounded by
propagating, step by step and to first order,
  * the rounding of a sum of m products in any order and blocking:
    gamma_m * sum |x_i y_i| (Higham, "Accuracy and Stability of Numerical
    Algorithms", the inner-product bound, gamma_m = m u / (1 - m u),
    u = 2^-24);
  * one rounding per elementwise operation (u times its magnitude);
  * the tanh / sigmoid evaluation, within 8 ulps of 1 in absolute terms;
  * the errors of the operands, through the derivative of each step
    (|d tanh(z/2)/dz| = (1 - h^2) / 2).
The bound is what the arithmetic allows in the worst case; a realistic fp32
evaluation is far inside it (the CPU pins check that it holds for an fp32
NumPy evaluation of the same formulas).
"""
from __future__ import annotations

import numpy as np
from scipy import sparse

U = 2.0 ** -24


def gamma(m: int) -> float:
    return m * U / (1.0 - m * U)


def _bf16_to_f64(bits):
    b = np.ascontiguousarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def grad_bound(q_bits, k_bits, q_pos, S, W, sigma, eps, eta, lam) -> np.ndarray:
    """Per-element bound [d, r] on |dW_fp32 - dW_exact|."""
    Q, K = _bf16_to_f64(q_bits), _bf16_to_f64(k_bits)
    W = np.asarray(W, np.float64)
    J, d = Q.shape
    n = K.shape[0]
    r = W.shape[1]
    aQ, aK, aW = np.abs(Q), np.abs(K), np.abs(W)
    # projections and the relaxed hash
    Zq, Zk = sigma * (Q @ W), sigma * (K @ W)
    eZq = abs(sigma) * gamma(d + 2) * (aQ @ aW)
    eZk = abs(sigma) * gamma(d + 2) * (aK @ aW)
    Hq, Hk = np.tanh(0.5 * Zq), np.tanh(0.5 * Zk)
    eHq = 0.5 * (1.0 - Hq * Hq) * eZq + 8 * U
    eHk = 0.5 * (1.0 - Hk * Hk) * eZk + 8 * U
    aHq, aHk = np.abs(Hq), np.abs(Hk)
    # label sums and products (labels are exact fp32 values)
    M = (np.arange(n)[None, :] <= np.asarray(q_pos)[:, None]).astype(np.float64)
    Sm = S * M
    aS = np.abs(Sm)
    rs, cs = Sm.sum(axis=1), Sm.sum(axis=0)
    e_rs, e_cs = gamma(n) * aS.sum(axis=1), gamma(J) * aS.sum(axis=0)
    P1 = Sm @ Hk
    eP1 = gamma(n) * (aS @ aHk) + aS @ eHk
    dHq = 2.0 * eps * (rs[:, None] * Hq - P1)
    edHq = 2.0 * abs(eps) * (e_rs[:, None] * aHq + np.abs(rs)[:, None] * eHq + eP1
                             + 3 * U * (np.abs(rs)[:, None] * aHq + np.abs(P1)))
    P2 = Sm.T @ Hq
    eP2 = gamma(J) * (aS.T @ aHq) + aS.T @ eHq
    C = M @ Hk
    eC = gamma(n) * (M @ aHk) + M @ eHk
    P3 = M.T @ C
    eP3 = gamma(J) * (M.T @ np.abs(C)) + M.T @ eC
    dHk = 2.0 * eps * (cs[:, None] * Hk - P2) + 2.0 * eta * P3
    edHk = (2.0 * abs(eps) * (e_cs[:, None] * aHk + np.abs(cs)[:, None] * eHk + eP2
                              + 3 * U * (np.abs(cs)[:, None] * aHk + np.abs(P2)))
            + 2.0 * abs(eta) * (eP3 + U * np.abs(P3)) + 2 * U * np.abs(dHk))
    # through the hash derivative
    gq, gk = 0.5 * (1.0 - Hq * Hq), 0.5 * (1.0 - Hk * Hk)
    dZq, dZk = dHq * gq, dHk * gk
    edZq = edHq * gq + np.abs(dHq) * aHq * eHq + 2 * U * np.abs(dZq)
    edZk = edHk * gk + np.abs(dHk) * aHk * eHk + 2 * U * np.abs(dZk)
    # the gradient products
    G1 = sigma * (Q.T @ dZq + K.T @ dZk)
    eG1 = abs(sigma) * (gamma(J + n + 1) * (aQ.T @ np.abs(dZq) + aK.T @ np.abs(dZk))
                        + aQ.T @ edZq + aK.T @ edZk)
    # decorrelation
    A = W.T @ W - np.eye(r)
    eA = gamma(d + 1) * (aW.T @ aW)
    na = float(np.sqrt(np.sum(A * A)))
    eD = np.zeros_like(W)
    D = np.zeros_like(W)
    if na > 0:
        ena = float(np.sqrt(np.sum(eA * eA))) + gamma(r * r + 1) * na
        WA = W @ A
        eWA = gamma(r) * (aW @ np.abs(A)) + aW @ eA
        D = 2.0 * lam * WA / na
        eD = 2.0 * abs(lam) * (eWA / na + np.abs(WA) * ena / (na * na)) + 3 * U * np.abs(D)
    return eG1 + eD + U * np.abs(G1 + D)


def loss_bound(q_bits, k_bits, q_pos, S, W, sigma, eps, eta, lam) -> np.ndarray:
    """Bound on |loss_fp32 - loss_exact| for (total, similarity, balance,
    decorrelation), each term a sum of many products whose order the
    evaluation chooses."""
    Q, K = _bf16_to_f64(q_bits), _bf16_to_f64(k_bits)
    W = np.asarray(W, np.float64)
    J, d = Q.shape
    n = K.shape[0]
    r = W.shape[1]
    aW = np.abs(W)
    Hq, Hk = np.tanh(0.5 * sigma * (Q @ W)), np.tanh(0.5 * sigma * (K @ W))
    eHq = 0.5 * (1.0 - Hq * Hq) * abs(sigma) * gamma(d + 2) * (np.abs(Q) @ aW) + 8 * U
    eHk = 0.5 * (1.0 - Hk * Hk) * abs(sigma) * gamma(d + 2) * (np.abs(K) @ aW) + 8 * U
    sim_mag = sim_err = bal_mag = bal_err = 0.0
    for j in range(J):
        p = int(q_pos[j])
        diff = Hq[j][None, :] - Hk[:p + 1]
        ediff = eHq[j][None, :] + eHk[:p + 1]
        s = np.abs(S[j, :p + 1])
        sim_mag += float(np.sum(s * np.sum(diff * diff, axis=1)))
        sim_err += float(np.sum(s * np.sum(2 * np.abs(diff) * ediff, axis=1)))
        c = Hk[:p + 1].sum(axis=0)
        ec = gamma(p + 1) * np.abs(Hk[:p + 1]).sum(axis=0) + eHk[:p + 1].sum(axis=0)
        bal_mag += float(c @ c)
        bal_err += float(2 * np.abs(c) @ ec)
    sim_b = abs(eps) * (sim_err + gamma(n * r + J + 2) * sim_mag)
    bal_b = abs(eta) * (bal_err + gamma(J * r + 2) * bal_mag)
    A = W.T @ W - np.eye(r)
    na = float(np.sqrt(np.sum(A * A)))
    eA = gamma(d + 1) * (aW.T @ aW)
    dec_b = abs(lam) * (float(np.sqrt(np.sum(eA * eA))) + gamma(r * r + 2) * na)
    tot = sim_b + bal_b + dec_b + 3 * U * (abs(eps) * sim_mag + abs(eta) * bal_mag + abs(lam) * na)
    return np.array([tot, sim_b, bal_b, dec_b])


# ------------------------------------------------------------------ probabilistic
# The worst-case bound above adds every rounding with the same sign; over
# sums of thousands of terms that is far from any real evaluation.  The
# probabilistic model (Higham and Mary, "A new approach to probabilistic
# rounding error analysis", SIAM J. Sci. Comput. 41 (2019)) takes each
# elementary rounding error delta_e as an independent mean-zero random
# variable with |delta_e| <= beta_e (u times the magnitude of the value it
# rounds; for a partial sum, at most the sum of the magnitudes of its
# terms).  To first order the error of one gradient element is
# E = sum_e c_e delta_e, with c_e the derivative of that element with respect
# to the rounded quantity (an adjoint of the evaluation graph), and
# Hoeffding's inequality gives |E| <= LAM sqrt(sum_e c_e^2 beta_e^2) except
# with probability 2 exp(-LAM^2 / 2) (LAM = 6: 3e-8 per element).
#
# The adjoints are exact (no magnitude inequality between them), and a
# partial sum that feeds several outputs is one elementary error whose
# coefficient is the sum over its consumers -- the causal sums are evaluated
# through per-64-row chunk sums of H_k shared by every query past the chunk,
# and the suffix sums through one partial per chunk shared by its 64 rows, so
# both are modelled that way.  Sum lengths count one rounding per product and
# one per addition, plus the split-k and cross-lane additions.
LAM = 6.0
CHUNK = 64  # rows per chunk of the causal-mask sums


def _rev_cumsum(x):
    return np.cumsum(x[::-1], axis=0)[::-1]


def grad_bound_prob(q_bits, k_bits, q_pos, S, W, sigma, eps, eta, lam, col_block: int = 16) -> np.ndarray:
    """Per-element bound [d, r] on |dW_fp32 - dW_exact| under the
    probabilistic rounding model.  S must be zero past each query's position
    (as the oracle's labels are); sigma, eps, eta and lam are taken as exact
    (fp32-representable) values."""
    u = U
    Q, K = _bf16_to_f64(q_bits), _bf16_to_f64(k_bits)
    W = np.asarray(W, np.float64)
    S = np.asarray(S, np.float64)
    J, d = Q.shape
    n = K.shape[0]
    r = W.shape[1]
    pos = np.clip(np.asarray(q_pos, np.int64), 0, n - 1)
    aQ, aK, aW, aS = np.abs(Q), np.abs(K), np.abs(W), np.abs(S)
    Q2, K2 = Q * Q, K * K
    # ---- exact values
    Hq, Hk = np.tanh(0.5 * sigma * (Q @ W)), np.tanh(0.5 * sigma * (K @ W))
    gq, gk = 0.5 * (1 - Hq * Hq), 0.5 * (1 - Hk * Hk)
    rs, cs = S.sum(axis=1), S.sum(axis=0)
    P1, P2 = S @ Hk, S.T @ Hq
    cum = np.cumsum(Hk, axis=0)
    C = cum[pos]                                   # M Hk
    Y = np.zeros((n, r))
    np.add.at(Y, pos, C)
    P3 = _rev_cumsum(Y)                            # M^T C
    dHq = 2 * eps * (rs[:, None] * Hq - P1)
    dHk = 2 * eps * (cs[:, None] * Hk - P2) + 2 * eta * P3
    dZq, dZk = dHq * gq, dHk * gk
    G1 = sigma * (Q.T @ dZq + K.T @ dZk)
    # ---- squared bounds beta^2 of the elementary errors, per (row, column)
    bHq = (2 * gq) ** 2 * ((0.5 * sigma) ** 2 * (2 * d + 1) * u * u * (aQ @ aW) ** 2) + (8 * u * Hq) ** 2
    bHk = (2 * gk) ** 2 * ((0.5 * sigma) ** 2 * (2 * d + 1) * u * u * (aK @ aW) ** 2) + (8 * u * Hk) ** 2
    bP1 = 2 * (n + 16) * u * u * (aS @ np.abs(Hk)) ** 2
    bP2 = 2 * (J + 16) * u * u * (aS.T @ np.abs(Hq)) ** 2
    brs = (n + 8) * u * u * aS.sum(axis=1) ** 2
    bcs = (J + 20) * u * u * aS.sum(axis=0) ** 2
    nb = (n + CHUNK - 1) // CHUNK
    chunk_of_row = np.arange(n) // CHUNK
    aHk_chunk = np.zeros((nb, r))
    np.add.at(aHk_chunk, chunk_of_row, np.abs(Hk))
    bT = (CHUNK + 3) * u * u * aHk_chunk ** 2                          # chunk sums of Hk
    cj = pos // CHUNK
    bC = (cj + CHUNK + 3)[:, None] * u * u * np.cumsum(np.abs(Hk), axis=0)[pos] ** 2
    aCpos = np.zeros((n, r))
    np.add.at(aCpos, pos, np.abs(C))
    aC_from = _rev_cumsum(aCpos)                  # sum of |C_j| over p_j >= i
    chunk_end = np.minimum(n, (np.arange(nb) + 1) * CHUNK)
    past_mag = np.vstack([aC_from[chunk_end[:-1]], np.zeros((1, r))]) if nb > 1 else np.zeros((1, r))
    bpast = (J + 3) * u * u * past_mag ** 2                            # per-chunk past-query partial
    nin = np.bincount(cj, minlength=nb)
    bP3 = (nin[chunk_of_row] + 1)[:, None] * u * u * aC_from ** 2
    ew = lambda dH, g, H, w, P, extra: (  # noqa: E731  elementwise dH, dZ roundings
        (2 * eps * g * w[:, None] * H) ** 2 + (2 * eps * g * (w[:, None] * H - P)) ** 2 + (g * dH) ** 2
        + (0.5 * dH * H * H) ** 2 + (0.5 * dH * (1 - H * H)) ** 2 + (g * dH) ** 2 + extra)
    bdZq = u * u * ew(dHq, gq, Hq, rs, P1, 0.0)
    bdZk = u * u * ew(dHk, gk, Hk, cs, P2, (2 * eta * gk * P3) ** 2 + (gk * dHk) ** 2)
    # ---- terms whose adjoint is a per-row scalar times a row of Q or K
    var = (sigma ** 2) * (Q2.T @ ((2 * eps * gq) ** 2 * bP1 + (2 * eps * Hq * gq) ** 2 * brs[:, None] + bdZq)
                          + K2.T @ ((2 * eps * gk) ** 2 * bP2 + (2 * eps * Hk * gk) ** 2 * bcs[:, None]
                                    + (2 * eta * gk) ** 2 * bP3 + bdZk))
    # final products (2 products of J and n terms, split-k, scale, accumulate)
    var += (2 * (J + n + 32) + 3) * u * u * (abs(sigma) * (aQ.T @ np.abs(dZq) + aK.T @ np.abs(dZk))) ** 2
    # ---- terms with full adjoints, a block of columns at a time
    # the causal mask, and the scatter of query rows onto their chunks
    Mmask = (np.arange(n)[None, :] <= pos[:, None]).astype(np.float64)
    scatter_chunk = sparse.csr_matrix((np.ones(J), (cj, np.arange(J))), shape=(nb, J))
    hq = -dHq * Hq + 2 * eps * rs[:, None] * gq     # d dZq / d Hq (direct)
    hk = -dHk * Hk + 2 * eps * cs[:, None] * gk     # d dZk / d Hk (direct)
    for c0 in range(0, r, col_block):
        c1 = min(r, c0 + col_block)
        w = c1 - c0
        # adjoints as [rows, w, d] (column c of the block, then the d outputs)
        aP3 = 2 * eta * sigma * gk[:, c0:c1, None] * K[:, None, :]
        aC = (Mmask @ aP3.reshape(n, w * d)).reshape(J, w, d) if eta != 0 else None  # M aP3
        aHq = sigma * hq[:, c0:c1, None] * Q[:, None, :]
        aHk = sigma * hk[:, c0:c1, None] * K[:, None, :]
        if eps != 0:
            aP2 = -2 * eps * sigma * gk[:, c0:c1, None] * K[:, None, :]
            aP1 = -2 * eps * sigma * gq[:, c0:c1, None] * Q[:, None, :]
            aHq += (S @ aP2.reshape(n, w * d)).reshape(J, w, d)
            aHk += (S.T @ aP1.reshape(J, w * d)).reshape(n, w, d)
        if eta != 0:
            aCf = aC.reshape(J, w * d)
            aHk += (Mmask.T @ aCf).reshape(n, w, d)                  # M^T aC
            # chunk sums T_b: consumed by every query whose chunk is past b
            byc = (scatter_chunk @ aCf).reshape(nb, w, d)
            aT = np.concatenate([_rev_cumsum(byc)[1:], np.zeros((1, w, d))])
            # per-chunk past partial of the suffix sums: consumed by the chunk's rows
            pad = np.zeros((nb * CHUNK, w, d))
            pad[:n] = aP3
            apast = pad.reshape(nb, CHUNK, w, d).sum(axis=1)
            var[:, c0:c1] += np.einsum("bwd,bw->dw", aT * aT, bT[:, c0:c1])
            var[:, c0:c1] += np.einsum("jwd,jw->dw", aC * aC, bC[:, c0:c1])
            var[:, c0:c1] += np.einsum("bwd,bw->dw", apast * apast, bpast[:, c0:c1])
        var[:, c0:c1] += np.einsum("jwd,jw->dw", aHq * aHq, bHq[:, c0:c1])
        var[:, c0:c1] += np.einsum("iwd,iw->dw", aHk * aHk, bHk[:, c0:c1])
    G = G1
    # ---- decorrelation fac * W A, fac = 2 lam / ||A||_F, A = W^T W - I
    A = W.T @ W - np.eye(r)
    na = float(np.sqrt(np.sum(A * A)))
    if na > 0 and lam != 0:
        fac = 2 * lam / na
        WA = W @ A
        bgram = (2 * d + 1) * u * u * (aW.T @ aW) ** 2              # [r, r]
        s_all = float(np.sum(A * A * bgram))
        # gram[e, f] enters WA[a, c] when f == c (coefficient fac W[a, e]) and
        # the norm for every output (coefficient -fac WA[a, c] A[e, f] / na^2)
        t = fac * WA / na ** 2                                      # [d, r]
        var += t * t * s_all
        cross = (fac * W)[:, :, None] - t[:, None, :] * A[None, :, :]  # [d, e, c]
        var += np.einsum("aec,ec->ac", cross ** 2 - (t[:, None, :] * A[None, :, :]) ** 2, bgram)
        var += fac ** 2 * 2 * (r + 1) * u * u * (aW @ np.abs(A)) ** 2   # W A products
        var += (fac * WA) ** 2 * u * u * (r * r / 2.0 + 3)            # norm, sqrt, 2 lam / na
        G = G1 + fac * WA
    var += 2 * u * u * (np.abs(G1) + np.abs(G - G1)) ** 2           # the final add
    return LAM * np.sqrt(var)


def loss_bound_prob(q_bits, k_bits, q_pos, S, W, sigma, eps, eta, lam) -> np.ndarray:
    """Bound on |loss_fp32 - loss_exact| for (total, similarity, balance,
    decorrelation) under the same probabilistic model, for an evaluation
    that forms the similarity term from its expansion
    sum_j S_j ||h_q||^2 - 2 h_q . (S h_k)_j + sum_i (S^T 1)_i ||h_k||^2 and the
    balance term from the causal sums (M h_k)_j (chunked as in the gradient).
    The derivative of the loss with respect to H_q, H_k is the dH of the
    gradient, so the hash errors enter with exactly those coefficients."""
    u = U
    Q, K = _bf16_to_f64(q_bits), _bf16_to_f64(k_bits)
    W = np.asarray(W, np.float64)
    S = np.asarray(S, np.float64)
    J, d = Q.shape
    n = K.shape[0]
    r = W.shape[1]
    pos = np.clip(np.asarray(q_pos, np.int64), 0, n - 1)
    aQ, aK, aW, aS = np.abs(Q), np.abs(K), np.abs(W), np.abs(S)
    Hq, Hk = np.tanh(0.5 * sigma * (Q @ W)), np.tanh(0.5 * sigma * (K @ W))
    gq, gk = 0.5 * (1 - Hq * Hq), 0.5 * (1 - Hk * Hk)
    rs, cs = S.sum(axis=1), S.sum(axis=0)
    P1, P2 = S @ Hk, S.T @ Hq
    C = np.cumsum(Hk, axis=0)[pos]
    Y = np.zeros((n, r))
    np.add.at(Y, pos, C)
    P3 = _rev_cumsum(Y)
    bHq = (2 * gq) ** 2 * ((0.5 * sigma) ** 2 * (2 * d + 1) * u * u * (aQ @ aW) ** 2) + (8 * u * Hq) ** 2
    bHk = (2 * gk) ** 2 * ((0.5 * sigma) ** 2 * (2 * d + 1) * u * u * (aK @ aW) ** 2) + (8 * u * Hk) ** 2
    bP1 = 2 * (n + 16) * u * u * (aS @ np.abs(Hk)) ** 2
    brs = (n + 8) * u * u * aS.sum(axis=1) ** 2
    bcs = (J + 20) * u * u * aS.sum(axis=0) ** 2
    nq, nk = (Hq * Hq).sum(axis=1), (Hk * Hk).sum(axis=1)
    a1, a2, pk = rs * nq, (Hq * P1).sum(axis=1), cs * nk
    sim = eps * (a1.sum() - 2 * a2.sum() + pk.sum())
    red = lambda m: (m / 1024.0 + 12) * u * u  # noqa: E731  strided partial sums, then a tree of 1024
    v_sim = eps ** 2 * (
        np.sum((2 * (rs[:, None] * Hq - P1)) ** 2 * bHq) + np.sum((2 * (cs[:, None] * Hk - P2)) ** 2 * bHk)
        + np.sum(nq ** 2 * brs) + np.sum(nk ** 2 * bcs) + np.sum((2 * Hq) ** 2 * bP1)
        + np.sum((3 * r + 16) * u * u * (np.abs(rs) * nq) ** 2)
        + 4 * np.sum((2 * r + 16) * u * u * ((np.abs(Hq) * np.abs(P1)).sum(axis=1)) ** 2)
        + np.sum((3 * r + 16) * u * u * (np.abs(cs) * nk) ** 2)
        + red(J) * (np.abs(a1).sum() + 2 * np.abs(a2).sum()) ** 2 + red(n) * np.abs(pk).sum() ** 2) \
        + 2 * u * u * sim ** 2
    # balance: causal sums with shared chunk partials
    nb = (n + CHUNK - 1) // CHUNK
    cj = pos // CHUNK
    aHk_chunk = np.zeros((nb, r))
    np.add.at(aHk_chunk, np.arange(n) // CHUNK, np.abs(Hk))
    bT = (CHUNK + 3) * u * u * aHk_chunk ** 2
    bC = (cj + CHUNK + 3)[:, None] * u * u * np.cumsum(np.abs(Hk), axis=0)[pos] ** 2
    byc = np.zeros((nb, r))
    np.add.at(byc, cj, 2 * C)
    cT = np.concatenate([_rev_cumsum(byc)[1:], np.zeros((1, r))])
    nc = (C * C).sum(axis=1)
    bal = eta * nc.sum()
    v_bal = eta ** 2 * (np.sum((2 * P3) ** 2 * bHk) + np.sum((2 * C) ** 2 * bC) + np.sum(cT ** 2 * bT)
                        + np.sum((2 * r + 16) * u * u * nc ** 2) + red(J) * nc.sum() ** 2) + u * u * bal ** 2
    # decorrelation lam ||A||_F
    A = W.T @ W - np.eye(r)
    na = float(np.sqrt(np.sum(A * A)))
    bgram = (2 * d + 1) * u * u * (aW.T @ aW) ** 2
    v_dec = (lam ** 2 * float(np.sum((A / na) ** 2 * bgram)) + (lam * na) ** 2 * u * u * (r * r / 2.0 + 3)
             if na > 0 else 0.0)
    # the total: the hash errors of the similarity and balance terms share their deltas
    v_tot = (v_sim + v_bal + v_dec
             + 2 * eps * eta * np.sum((2 * (cs[:, None] * Hk - P2)) * (2 * P3) * bHk)
             + 2 * u * u * (abs(sim) + abs(bal) + abs(lam) * na) ** 2)
    v_tot = max(v_tot, 0.0)
    return LAM * np.sqrt(np.array([v_tot, v_sim, v_bal, v_dec]))
