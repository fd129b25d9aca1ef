"""CPU oracle for the HATA decode step -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package.  The HIP library never loads it and shares no
code with it; inputs reach both sides from the seeded generators alone.

Two independent implementations live here:

* ``hata_oracle.c`` (plain C, fp32 projection with -ffp-contract=off, loop
  popcount, qsort top-k, fp64 attention), wrapped below with ctypes;
* ``brute.py`` (pure Python bit loops and ``sorted``) for tiny shapes.

Both follow the paper notes on "HATA: Trainable and Hardware-Efficient
Hash-Aware Top-k Attention for Scalable Large Model Inference", section
"Key design" (subsections "Learning-to-Hash modelling" and "Decode-stage
algorithm") and section "Overall framework".  The readings taken where the
notes are silent are stated in ``hata_oracle.c``.

Parity status of each function: pinned by tests/test_oracle_pins.py (closed
forms, exact-arithmetic cases, invariants, library routines, brute force);
none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hata_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# -ffp-contract=off: one rounded product and one rounded add per term, in the
# order the source states.  -fno-fast-math keeps IEEE semantics.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (no GPU toolchain involved)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.oracle_encode_rows.argtypes = [P, i64, ctypes.c_int, P, ctypes.c_int, P, P]
        L.oracle_encode_rows.restype = None
        L.oracle_popcount64.argtypes = [ctypes.c_uint64]
        L.oracle_popcount64.restype = ctypes.c_int
        L.oracle_hamming_gqa.argtypes = [P, ctypes.c_int, P, i64, ctypes.c_int, P]
        L.oracle_hamming_gqa.restype = None
        L.oracle_topk.argtypes = [P, i64, ctypes.c_int, P]
        L.oracle_topk.restype = ctypes.c_int
        L.oracle_attention.argtypes = [P, ctypes.c_int, P, P, P, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_float, P]
        L.oracle_attention.restype = None
        L.oracle_decode_step.argtypes = [P, P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, i64, P, ctypes.c_int,
                                         ctypes.c_float, P, P, P, P, ctypes.c_int]
        L.oracle_decode_step.restype = ctypes.c_int
        L.oracle_dense_attention.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, i64, P, ctypes.c_float, P, ctypes.c_int]
        L.oracle_dense_attention.restype = ctypes.c_int
        L.oracle_max_threads.argtypes = []
        L.oracle_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def encode(x_bf16: np.ndarray, W: np.ndarray, return_proj: bool = False):
    """HashEncode rows x (bf16 bits, [..., d]) with W [d, r] -> uint64 [..., r/64]."""
    x = _c(x_bf16, np.uint16)
    W = _c(W, np.float32)
    d, r = W.shape
    assert x.shape[-1] == d and r >= 1
    rows = int(np.prod(x.shape[:-1], dtype=np.int64))
    codes = np.zeros(x.shape[:-1] + ((r + 63) // 64,), np.uint64)
    proj = np.zeros(x.shape[:-1] + (r,), np.float32) if return_proj else None
    lib().oracle_encode_rows(_p(x), rows, d, _p(W), r, _p(codes), _p(proj))
    return (codes, proj) if return_proj else codes


def popcount64(v: int) -> int:
    return lib().oracle_popcount64(ctypes.c_uint64(int(v)))


def hamming_gqa(qcodes: np.ndarray, kcodes: np.ndarray) -> np.ndarray:
    """qcodes [G, words], kcodes [n, words] -> int32 [n] summed distances."""
    qc = _c(qcodes, np.uint64)
    kc = _c(kcodes, np.uint64)
    G, words = qc.shape
    n = kc.shape[0]
    assert kc.shape[1] == words
    S = np.zeros(n, np.int32)
    lib().oracle_hamming_gqa(_p(qc), G, _p(kc), n, words, _p(S))
    return S


def topk(S: np.ndarray, k: int) -> np.ndarray:
    """int32 [k]: ascending ids of the k smallest (score, id); -1 padded."""
    S = _c(S, np.int32)
    idx = np.empty(k, np.int32)
    m = lib().oracle_topk(_p(S), S.shape[0], k, _p(idx))
    if m < 0:
        raise MemoryError("oracle_topk allocation failed")
    return idx


def attention(q_bf16: np.ndarray, K_bf16: np.ndarray, V_bf16: np.ndarray,
              idx: np.ndarray, scale: float) -> np.ndarray:
    """q [G, d]; K, V [n, d] (one KV head); idx [m] (-1 skipped) -> fp32 [G, d]."""
    q = _c(q_bf16, np.uint16)
    K = _c(K_bf16, np.uint16)
    V = _c(V_bf16, np.uint16)
    idx = _c(idx, np.int32)
    G, d = q.shape
    out = np.zeros((G, d), np.float32)
    lib().oracle_attention(_p(q), G, _p(K), _p(V), _p(idx), idx.shape[0], d,
                           ctypes.c_float(scale), _p(out))
    return out


def decode_step(q, K, V, W, codes, seq_lens, k, scale, nthreads: int = 0,
                want_scores: bool = False, want_qcodes: bool = False, Wk=None):
    """Whole decode step over every (sequence, KV head) unit.

    q [B,Hq,d] bf16 bits; K, V [B,Hkv,cap,d] bf16 bits; W [Hkv,d,r] fp32;
    codes [B,Hkv,cap,r/64] uint64, rows < n_b-1 valid -- a copy is returned
    with row n_b-1 appended.  Wk (optional, like W): a separate key encoder
    for the appended row (HashAttention summary page, "Approach": independent
    query and key encoders); None means W encodes both.
    Returns dict(out, idx, codes[, scores][, qcodes]).
    """
    q = _c(q, np.uint16)
    K = _c(K, np.uint16)
    V = _c(V, np.uint16)
    W = _c(W, np.float32)
    codes = np.array(codes, dtype=np.uint64, copy=True, order="C")
    seq = _c(seq_lens, np.int32)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = K.shape
    r = W.shape[2]
    out = np.zeros((B, Hq, d), np.float32)
    idx = np.zeros((B, Hkv, k), np.int32)
    scores = np.full((B, Hkv, cap), -1, np.int32) if want_scores else None
    qcodes = np.zeros((B, Hq, (r + 63) // 64), np.uint64) if want_qcodes else None
    Wk = None if Wk is None else _c(Wk, np.float32)
    if Wk is not None and Wk.shape != W.shape:
        raise ValueError("Wk must have W's shape")
    rc = lib().oracle_decode_step(_p(q), _p(K), _p(V), _p(W), _p(Wk), _p(codes), B, Hq, Hkv, d, r,
                                  cap, _p(seq), k, ctypes.c_float(scale), _p(out), _p(idx),
                                  _p(scores), _p(qcodes), nthreads)
    if rc != 0:
        raise ValueError("oracle_decode_step rejected its arguments")
    res = {"out": out, "idx": idx, "codes": codes}
    if want_scores:
        res["scores"] = scores
    if want_qcodes:
        res["qcodes"] = qcodes
    return res


def dense_attention(q, K, V, seq_lens, scale, nthreads: int = 0) -> np.ndarray:
    q = _c(q, np.uint16)
    K = _c(K, np.uint16)
    V = _c(V, np.uint16)
    seq = _c(seq_lens, np.int32)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = K.shape
    out = np.zeros((B, Hq, d), np.float32)
    rc = lib().oracle_dense_attention(_p(q), _p(K), _p(V), B, Hq, Hkv, d, cap, _p(seq),
                                      ctypes.c_float(scale), _p(out), nthreads)
    if rc != 0:
        raise ValueError("oracle_dense_attention rejected its arguments")
    return out


def build_cache(K, W, seq_lens=None) -> np.ndarray:
    """Prefill-side code cache: encode every row of K [B,Hkv,cap,d] with its
    KV head's W (rows beyond seq_lens[b] stay 0)."""
    K = _c(K, np.uint16)
    B, Hkv, cap, d = K.shape
    r = W.shape[2]
    codes = np.zeros((B, Hkv, cap, (r + 63) // 64), np.uint64)
    for b in range(B):
        n = cap if seq_lens is None else int(seq_lens[b])
        for h in range(Hkv):
            codes[b, h, :n] = encode(K[b, h, :n], W[h])
    return codes


def max_threads() -> int:
    return lib().oracle_max_threads()
