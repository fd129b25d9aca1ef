"""Pure-Python brute force of the HATA decode step, for tiny shapes only.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``).  It is a
second, independent implementation of the steps in the paper notes on HATA,
section "Key design: Decode-stage algorithm": HashEncode (projection, sign,
bit-pack), append, Hamming distance as the count of differing bits, GQA sum,
top-k by sorting, exact softmax attention over the kept rows.

Everything is a Python loop: bits are tested one at a time, the sort is
``sorted``, exp is ``math.exp`` on Python floats (fp64).  The only concession
to bit-exactness with the fp32 projection is that each product and partial sum
is rounded to fp32 with ``numpy.float32``, in increasing input index.
"""
from __future__ import annotations

import math
import struct

import numpy as np


def bf16_bits_to_float(h: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(h) & 0xFFFF) << 16))[0]


def project(x_bits, W) -> list:
    """fp32 projection p_c = sum_i x_i W[i][c], rounded per operation."""
    d = len(x_bits)
    r = len(W[0])
    xs = [np.float32(bf16_bits_to_float(v)) for v in x_bits]
    out = []
    for c in range(r):
        acc = np.float32(0.0)
        for i in range(d):
            acc = np.float32(acc + np.float32(xs[i] * np.float32(W[i][c])))
        out.append(acc)
    return out


def encode(x_bits, W) -> list:
    """List of r/64 Python ints; bit c of the code is bit c%64 of word c//64."""
    p = project(x_bits, W)
    r = len(p)
    words = [0] * ((r + 63) // 64)
    for c in range(r):
        if p[c] >= 0.0:
            words[c // 64] += 1 << (c % 64)
    return words


def hamming(a_words, b_words) -> int:
    """Number of bit positions where the two codes differ, one bit at a time."""
    n = 0
    for a, b in zip(a_words, b_words):
        for bit in range(64):
            if ((a >> bit) & 1) != ((b >> bit) & 1):
                n += 1
    return n


def topk(S, k) -> list:
    order = sorted(range(len(S)), key=lambda i: (S[i], i))
    kept = sorted(order[:k])
    return kept + [-1] * (k - len(kept))


def attention(q_rows, K_rows, V_rows, idx, scale) -> list:
    kept = [i for i in idx if i >= 0]
    outs = []
    for q in q_rows:
        qf = [bf16_bits_to_float(v) for v in q]
        z = []
        for i in kept:
            kf = [bf16_bits_to_float(v) for v in K_rows[i]]
            z.append(scale * sum(a * b for a, b in zip(qf, kf)))
        m = max(z)
        w = [math.exp(t - m) for t in z]
        den = sum(w)
        d = len(qf)
        acc = [0.0] * d
        for wi, i in zip(w, kept):
            vf = [bf16_bits_to_float(v) for v in V_rows[i]]
            for c in range(d):
                acc[c] += wi * vf[c]
        outs.append([a / den for a in acc])
    return outs


def decode_step(q, K, V, W, codes, seq_lens, k, scale):
    """Same contract as oracle.decode_step, on nested lists / small arrays.

    q [B][Hq][d]; K, V [B][Hkv][cap][d] (bf16 bits); W [Hkv][d][r] floats;
    codes [B][Hkv][cap][words] ints (rows < n_b-1 valid).
    Returns (out [B][Hq][d] floats, idx [B][Hkv][k], codes, scores).
    """
    B = len(q)
    Hq = len(q[0])
    Hkv = len(K[0])
    G = Hq // Hkv
    codes = [[[list(row) for row in head] for head in seq] for seq in codes]
    out = [[None] * Hq for _ in range(B)]
    idx_all = [[None] * Hkv for _ in range(B)]
    scores = [[None] * Hkv for _ in range(B)]
    for b in range(B):
        n = int(seq_lens[b])
        for h in range(Hkv):
            Wh = W[h]
            qc = [encode(q[b][h * G + g], Wh) for g in range(G)]
            codes[b][h][n - 1] = encode(K[b][h][n - 1], Wh)
            S = [sum(hamming(qc[g], codes[b][h][i]) for g in range(G)) for i in range(n)]
            idx = topk(S, k)
            o = attention([q[b][h * G + g] for g in range(G)], K[b][h], V[b][h], idx, scale)
            for g in range(G):
                out[b][h * G + g] = o[g]
            idx_all[b][h] = idx
            scores[b][h] = S
    return out, idx_all, codes, scores
