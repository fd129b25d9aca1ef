"""Seeded synthetic inputs for the HATA decode step.

This module draws inputs only: it holds none of the method's arithmetic and
is shared by the tests, the benchmark and the smoke check (for both the HIP
path and the CPU oracle).  Everything is numpy ``Generator(PCG64(seed))``;
fp32 draws are rounded to bf16 bit patterns with round-to-nearest-even.

Workload shapes follow the paper notes on HATA: Llama-shaped attention layers
(section "Experiments": Llama-2-7B is multi-head with 32 heads, Llama-3.1-8B
uses GQA with 32 query heads over 8 KV heads, head dim 128), 128-bit codes
(section "Key findings": 128 bits is the usual balance), and a fixed budget
of 512 tokens (section "Limitations").  Needle-in-a-haystack accuracy
(section "Experiments", NIAH table) is stood in for by planted keys close to
the queries; no benchmark item is used.

Recipes (the readings are listed in the repository's design notes):

* exact  -- q/K/V = a/8 with a uniform in {-32..32}; W_H uniform in {-1,0,+1}.
            Every partial sum of a projection is a multiple of 1/8 of magnitude
            at most 512, so fp32 projections are exact in any order.
* gauss  -- q/K/V ~ N(0,1); W_H ~ N(0, 1/128) per KV head; `outliers` key
            channels per KV head (chosen from the layer seed) scaled x8;
            `needles` planted keys per (sequence, KV head) at distinct
            positions in [0, n-1): 0.9*q_g + e, e ~ N(0, 0.19), g cycling over
            the group's query heads, written after outlier scaling.
* Seeds: layer seed (W_H, outlier channels) and one seed per sequence;
  per sequence the draw order is K, V, q, needle positions, needle noise.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
from dataclasses import dataclass, field

import numpy as np

D = 128
R = 128


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint32, copy=True)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact widening)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Shape:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    k: int
    dist: str            # "exact" | "gauss"
    seed_base: int       # layer seed = seed_base + 999, sequence b seed = seed_base + b
    outliers: int = 0
    needles: int = 0
    d: int = D
    r: int = R

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def units(self) -> int:
        return self.B * self.Hkv

    def scaled(self, **kw) -> "Shape":
        args = dict(self.__dict__)
        args.update(kw)
        return Shape(**args)


# The five workloads (one decode step of one attention layer each).
CONFIGS = {
    1: Shape("tiny-exact-gqa4-4k", B=1, Hq=4, Hkv=1, N=4096, k=256, dist="exact", seed_base=1000),
    2: Shape("llama3.1-8b-layer-32k", B=1, Hq=32, Hkv=8, N=32768, k=512, dist="gauss",
             seed_base=2000, outliers=4, needles=16),
    3: Shape("llama3.1-8b-layer-64k-b4", B=4, Hq=32, Hkv=8, N=65536, k=512, dist="gauss",
             seed_base=3000, outliers=4, needles=16),
    4: Shape("llama3.1-8b-layer-128k", B=1, Hq=32, Hkv=8, N=131072, k=512, dist="gauss",
             seed_base=4000, outliers=4),
    5: Shape("llama2-7b-mha-layer-32k-b8", B=8, Hq=32, Hkv=32, N=32768, k=512, dist="gauss",
             seed_base=5000, outliers=4),
}


@dataclass
class Inputs:
    shape: Shape
    q: np.ndarray          # uint16 [B, Hq, d]      (bf16 bits)
    K: np.ndarray          # uint16 [B, Hkv, cap, d]
    V: np.ndarray          # uint16 [B, Hkv, cap, d]
    W: np.ndarray          # float32 [Hkv, d, r]
    seq_lens: np.ndarray   # int32 [B]
    k: int
    scale: float
    needle_pos: np.ndarray = field(default=None)  # int32 [B, Hkv, needles] or None
    outlier_ch: np.ndarray = field(default=None)  # int32 [Hkv, outliers] or None

    @property
    def cap(self) -> int:
        return self.K.shape[2]


def _exact_vals(rng, size) -> np.ndarray:
    a = rng.integers(-32, 33, size=size, dtype=np.int32)
    return bf16_bits(a.astype(np.float32) / np.float32(8.0))


def _gauss_bits(rng, size) -> np.ndarray:
    return bf16_bits(rng.standard_normal(size, dtype=np.float32))


def make_inputs(shape: Shape, cap: int | None = None, seq_lens=None, k: int | None = None,
                scale: float | None = None) -> Inputs:
    """Draw one layer's decode-step inputs.  Rows >= seq_lens[b] (up to cap)
    are drawn too, so a larger cap only adds rows past the valid range."""
    B, Hq, Hkv, d, r = shape.B, shape.Hq, shape.Hkv, shape.d, shape.r
    G = shape.G
    N = shape.N
    cap = N if cap is None else int(cap)
    if seq_lens is None:
        seq_lens = np.full(B, N, np.int32)
    seq_lens = np.asarray(seq_lens, np.int32)
    assert seq_lens.shape == (B,) and (seq_lens >= 1).all() and (seq_lens <= cap).all()
    k = shape.k if k is None else int(k)
    scale = (1.0 / np.sqrt(d)) if scale is None else float(scale)

    lrng = np.random.Generator(np.random.PCG64(shape.seed_base + 999))
    if shape.dist == "exact":
        W = lrng.integers(-1, 2, size=(Hkv, d, r), dtype=np.int32).astype(np.float32)
        outlier_ch = None
    else:
        W = (lrng.standard_normal((Hkv, d, r), dtype=np.float32)
             * np.float32(1.0 / np.sqrt(128.0))).astype(np.float32)
        outlier_ch = (np.stack([lrng.choice(d, size=shape.outliers, replace=False)
                                for _ in range(Hkv)]).astype(np.int32)
                      if shape.outliers else None)

    q = np.empty((B, Hq, d), np.uint16)
    K = np.empty((B, Hkv, cap, d), np.uint16)
    V = np.empty((B, Hkv, cap, d), np.uint16)
    needle_pos = np.zeros((B, Hkv, shape.needles), np.int32) if shape.needles else None

    def draw(b: int) -> None:
        # sequence b: its own generator, its own slices of q, K, V
        rng = np.random.Generator(np.random.PCG64(shape.seed_base + b))
        if shape.dist == "exact":
            K[b] = _exact_vals(rng, (Hkv, cap, d))
            V[b] = _exact_vals(rng, (Hkv, cap, d))
            q[b] = _exact_vals(rng, (Hq, d))
            return
        # K is drawn in fp32 per head so outliers and needles are applied
        # before the single bf16 rounding.
        for h in range(Hkv):
            Kh = rng.standard_normal((cap, d), dtype=np.float32)
            if outlier_ch is not None:
                Kh[:, outlier_ch[h]] *= np.float32(8.0)
            K[b, h] = bf16_bits(Kh)
            del Kh
        for h in range(Hkv):
            V[b, h] = _gauss_bits(rng, (cap, d))
        qf = rng.standard_normal((Hq, d), dtype=np.float32)
        q[b] = bf16_bits(qf)
        if shape.needles:
            n = int(seq_lens[b])
            m = min(shape.needles, max(n - 1, 0))
            for h in range(Hkv):
                pos = np.sort(rng.choice(max(n - 1, 1), size=m, replace=False)).astype(np.int32)
                noise = rng.standard_normal((m, d), dtype=np.float32) * np.float32(np.sqrt(0.19))
                qsrc = bf16_to_f32(q[b, h * G + (np.arange(m) % G)])
                K[b, h, pos] = bf16_bits(np.float32(0.9) * qsrc + noise)
                needle_pos[b, h, :m] = pos
                needle_pos[b, h, m:] = -1

    # sequences are independent draws: large batches fill on several threads
    # (the values do not depend on the thread count)
    workers = min(B, os.cpu_count() or 1, 16)
    if workers > 1 and B * Hkv * cap * d >= (1 << 24):
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(draw, range(B)))
    else:
        for b in range(B):
            draw(b)
    return Inputs(shape=shape, q=q, K=K, V=V, W=W, seq_lens=seq_lens, k=k, scale=scale,
                  needle_pos=needle_pos, outlier_ch=outlier_ch)


def small_shape(B=1, Hq=4, Hkv=1, N=300, k=16, dist="gauss", seed_base=7000,
                outliers=0, needles=0) -> Shape:
    """Ad-hoc shape for parity tests (the recipes above, any size)."""
    return Shape(f"adhoc-b{B}-hq{Hq}-hkv{Hkv}-n{N}-k{k}-{dist}", B=B, Hq=Hq, Hkv=Hkv, N=N, k=k,
                 dist=dist, seed_base=seed_base, outliers=outliers, needles=needles)
