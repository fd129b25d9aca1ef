"""Shared helpers of the GPU parity tests: upload seeded inputs, run the
oracle stage by stage on the GPU's own codes (so allowed sign flips in the
encode cannot cascade), and compare with the stated bars."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from hash_top_sparse_amd import synth

# Attention tolerance, per element: |gpu - ref| <= ATOL + RTOL * |ref|
# (max-abs 2e-3 and max-rel 1e-3 in fp32, in allclose form so that outputs
# near zero are judged by the absolute bar).
ATOL = 2e-3
RTOL = 1e-3
# Encode on inputs whose projections are not exact: a bit may differ from the
# oracle only where the oracle's projection is smaller than this in magnitude.
FLIP_EPS = 1e-4


def bf16_tensor(a: np.ndarray, dev="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def codes_tensor(a: np.ndarray, dev="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint64).view(np.int64)).to(dev)


def codes_np(t: torch.Tensor) -> np.ndarray:
    """Code rows as the oracle holds them: uint64 words, ceil(r/64) a row (a
    32-bit code row, held as one int32 word, zero-extended)."""
    a = t.cpu().numpy()
    if a.dtype == np.int32:
        return a.view(np.uint32).astype(np.uint64)
    return a.view(np.uint64)


def scores_np(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


class Dev:
    """Inputs of one decode step on the GPU."""

    def __init__(self, inp: synth.Inputs, dev="cuda"):
        self.inp = inp
        self.q = bf16_tensor(inp.q, dev)
        self.K = bf16_tensor(inp.K, dev)
        self.V = bf16_tensor(inp.V, dev)
        self.W = torch.from_numpy(inp.W).to(dev)
        self.seq = torch.from_numpy(inp.seq_lens.astype(np.int32)).to(dev)
        B, Hq, _ = inp.q.shape
        _, Hkv, cap, _ = inp.K.shape
        self.B, self.Hq, self.Hkv, self.cap = B, Hq, Hkv, cap
        self.max_len = int(inp.seq_lens.max())


def gpu_build_cache(hb, d: Dev) -> torch.Tensor:
    """Code cache for rows [0, cap) built by the library's encode (prefill)."""
    codes = torch.zeros((d.B, d.Hkv, d.cap, 2), dtype=torch.int64, device="cuda")
    hb.encode_append(d.K, d.W, codes, n_new=d.cap)
    return codes


def gpu_query_codes(hb, d: Dev) -> torch.Tensor:
    qc = torch.zeros((d.B, d.Hq, 1, 2), dtype=torch.int64, device="cuda")
    hb.encode_append(d.q.view(d.B, d.Hq, 1, 128), d.W, qc, n_new=1)
    return qc.view(d.B, d.Hq, 2)


def check_codes(gpu: np.ndarray, x_bits: np.ndarray, W: np.ndarray, exact: bool) -> int:
    """gpu codes [rows, 2] vs oracle encode of x_bits [rows, d] with W [d, r].
    Returns the number of (allowed) flipped bits; asserts on any other mismatch."""
    ref, proj = oracle.encode(x_bits, W, return_proj=True)
    if exact:
        np.testing.assert_array_equal(gpu, ref)
        return 0
    diff = gpu ^ ref
    if not diff.any():
        return 0
    rows, words = np.nonzero(diff)
    flips = 0
    for r_, w_ in zip(rows, words):
        v = int(diff[r_, w_])
        for bit in range(64):
            if (v >> bit) & 1:
                c = w_ * 64 + bit
                p = float(proj[r_, c])
                assert abs(p) < FLIP_EPS, f"bit {c} of row {r_} differs with |p| = {abs(p)}"
                flips += 1
    return flips


def oracle_units(inp: synth.Inputs, qcodes: np.ndarray, codes: np.ndarray, units=None):
    """Steps 3-5 of the oracle per unit on the given codes.
    qcodes [B,Hq,2]; codes [B,Hkv,cap,2] (row n-1 already appended).
    Returns (scores dict, idx [B,Hkv,k], out [B,Hq,d])."""
    B, Hq, d = inp.q.shape
    Hkv = inp.K.shape[1]
    G = Hq // Hkv
    k = inp.k
    idx = np.full((B, Hkv, k), -2, np.int32)
    out = np.full((B, Hq, d), np.nan, np.float32)
    scores = {}
    for b in range(B):
        n = int(inp.seq_lens[b])
        for h in range(Hkv):
            if units is not None and (b, h) not in units:
                continue
            S = oracle.hamming_gqa(qcodes[b, h * G:(h + 1) * G], codes[b, h, :n])
            scores[(b, h)] = S
            ix = oracle.topk(S, k)
            idx[b, h] = ix
            out[b, h * G:(h + 1) * G] = oracle.attention(inp.q[b, h * G:(h + 1) * G], inp.K[b, h, :n],
                                                         inp.V[b, h, :n], ix, inp.scale)
    return scores, idx, out


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str = "out"):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} elements outside tolerance; first at {tuple(i)}: "
                             f"gpu={gpu[tuple(i)]} ref={ref[tuple(i)]}")
    big = np.abs(ref) > 1e-2
    return float(err.max()), float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0


def paginate(x: torch.Tensor, P: int, bt: torch.Tensor, num_pages: int, fill=0) -> torch.Tensor:
    """x [B, Hkv, cap, C] -> pool [num_pages, Hkv, P, C] with page bt[b, i]
    holding rows [i P, (i + 1) P) of sequence b (unused pages keep `fill`)."""
    B, Hkv, cap, C = x.shape
    mp = bt.shape[1]
    xp = torch.full((B, Hkv, mp * P, C), fill, dtype=x.dtype, device=x.device)
    xp[:, :, :cap] = x
    pool = torch.full((num_pages, Hkv, P, C), fill, dtype=x.dtype, device=x.device)
    pool[bt.reshape(-1).long()] = xp.view(B, Hkv, mp, P, C).permute(0, 2, 1, 3, 4).reshape(B * mp, Hkv, P, C)
    return pool


def gather_pages(pool: torch.Tensor, bt: torch.Tensor, cap: int) -> torch.Tensor:
    num_pages, Hkv, P, C = pool.shape
    B, mp = bt.shape
    g = pool[bt.reshape(-1).long()].view(B, mp, Hkv, P, C).permute(0, 2, 1, 3, 4).reshape(B, Hkv, mp * P, C)
    return g[:, :, :cap]
