"""Oracle for the prefill step -- TEST INFRASTRUCTURE ONLY.

Only the test-suite and the benchmark's CPU leg may import this module; the
HIP library shares no code with it.  numpy in fp64.

Follows the HATA notes page, section "Method", "Overall framework", second
stage: during prefill the attention is computed as usual (causal scaled
dot-product softmax attention over the prompt) while the keys are encoded
into binary hash codes that go into the code cache.  The encode is the
decode path's HashEncode (oracle.encode / oracle.build_cache, pinned
elsewhere) applied to every prompt key.

Readings (listed in the design notes):
  * query i of a prompt of length L sits at position i and attends keys
    0..i of the same sequence (causal), with scale 1/sqrt(d) unless given;
  * query head j reads KV head j // G (contiguous groups), as in decode;
  * rows at positions >= L are neither read nor written.

Parity status: pinned in tests/test_oracle_prefill_pins.py by closed cases
(the first row is V[0]; equal logits give the running mean of V; a dominant
logit selects its V row), causality (later keys do not change earlier rows),
and the last row against the decode oracle's dense attention (a separate C
implementation) for every head.
"""
from __future__ import annotations

import numpy as np

import oracle


def _f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def causal_attention(q_bits, K_bits, V_bits, seq_lens, scale=None) -> np.ndarray:
    """q [B, Hq, S, d], K and V [B, Hkv, cap, d] (bf16 bits); returns fp64
    [B, Hq, S, d] with rows at positions >= seq_lens[b] left zero."""
    B, Hq, S, d = q_bits.shape
    Hkv = K_bits.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.zeros((B, Hq, S, d))
    for b in range(B):
        n = int(seq_lens[b])
        if n <= 0:
            continue
        future = np.triu(np.ones((n, n), dtype=bool), k=1)  # key index > query index
        for h in range(Hq):
            Q = _f64(q_bits[b, h, :n])
            Kh = _f64(K_bits[b, h // G, :n])
            Vh = _f64(V_bits[b, h // G, :n])
            logits = (Q @ Kh.T) * scale
            logits[future] = -np.inf
            logits -= logits.max(axis=1, keepdims=True)
            p = np.exp(logits)
            p /= p.sum(axis=1, keepdims=True)
            out[b, h, :n] = p @ Vh
    return out


def abs_weighted_values(q_bits, K_bits, V_bits, seq_lens, scale=None) -> np.ndarray:
    """The same softmax weights applied to |V|: sum_j p_ij |v_jc|.  Bounds the
    effect of rounding the weights before the value product."""
    B, Hq, S, d = q_bits.shape
    Hkv = K_bits.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.zeros((B, Hq, S, d))
    for b in range(B):
        n = int(seq_lens[b])
        if n <= 0:
            continue
        future = np.triu(np.ones((n, n), dtype=bool), k=1)
        for h in range(Hq):
            Q = _f64(q_bits[b, h, :n])
            Kh = _f64(K_bits[b, h // G, :n])
            logits = (Q @ Kh.T) * scale
            logits[future] = -np.inf
            logits -= logits.max(axis=1, keepdims=True)
            p = np.exp(logits)
            p /= p.sum(axis=1, keepdims=True)
            out[b, h, :n] = p @ np.abs(_f64(V_bits[b, h // G, :n]))
    return out


def attention_rows(q_rows_bits, positions, K_bits, V_bits, scale=None, with_abs=False):
    """Single rows of the same attention: query row m (bf16 bits [d]) at
    position positions[m] attends keys 0..positions[m] of K, V [n, d] (one
    KV head).  For sampled checks of long prompts.  with_abs also returns the
    weights applied to |V| (as abs_weighted_values)."""
    d = K_bits.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.zeros((len(positions), d))
    absw = np.zeros((len(positions), d))
    for m, i in enumerate(positions):
        i = int(i)
        Q = _f64(q_rows_bits[m])
        Kh = _f64(K_bits[:i + 1])
        logits = (Kh @ Q) * scale
        logits -= logits.max()
        p = np.exp(logits)
        p /= p.sum()
        Vh = _f64(V_bits[:i + 1])
        out[m] = p @ Vh
        absw[m] = p @ np.abs(Vh)
    return (out, absw) if with_abs else out


def prefill(q_bits, K_bits, V_bits, W, seq_lens, scale=None):
    """Attention output (fp64) and the code cache rows 0..L-1 of every
    (sequence, KV head), as oracle.build_cache lays them out."""
    out = causal_attention(q_bits, K_bits, V_bits, seq_lens, scale)
    codes = oracle.build_cache(K_bits, W, seq_lens)
    return out, codes
