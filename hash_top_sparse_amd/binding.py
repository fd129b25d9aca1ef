"""ctypes binding over libhata.so (see include/hata.h for the full contract).

Argument marshalling only: each function takes torch tensors that already
live on the GPU, derives the sizes from their shapes, passes raw device
pointers plus torch's current stream to the C entry point of the same name,
and raises HataError on a non-zero status.  Every step of the path runs in
the library's HIP kernels; there is no fallback.

dtype conventions on the torch side: bf16 arrays are torch.bfloat16; a code
row of r bits is r/32 32-bit words, held as torch.int32 [..., r/32] or, for
r >= 64, as torch.int64 [..., r/64] (the same bytes; `new_codes` makes the
int64 form for r >= 64 and the int32 one at r = 32); scores are torch.int16
holding uint16 values, indices are torch.int32.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhata.so")
TRACE_LIB_PATH = os.path.join(_HERE, "libhata_trace.so")

OP_TOPK = 1
OP_SPARSE_DECODE = 2
OP_DECODE_STEP = 3
OP_DENSE_DECODE = 4
OP_DECODE_STEP_PAGED = 5

_lib = None


class HataError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libhata.so (built in-tree by hash_top_sparse_amd/build.py).  The
    first call fixes the library: `path` may name the phase-trace build
    (libhata_trace.so) instead, for the phase measurement of bench.py."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m hash_top_sparse_amd.build`")
    L = ctypes.CDLL(path)
    P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "hata_status_string": ([I], ctypes.c_char_p),
        "hata_last_error_message": ([], ctypes.c_char_p),
        "hata_version": ([], I),
        "hata_encode_append": ([P, I64, I, I, I, P, I, I, I, P, I64, P, P], I),
        "hata_hamming_scores": ([P, P, I, I, I, I, I64, P, I64, P, P], I),
        "hata_topk": ([P, I, I, I64, P, I64, I, I, P, P, SZ, P], I),
        "hata_sparse_decode": ([P, P, P, I, I, I, I, I64, P, I, F, P, P, SZ, P], I),
        "hata_decode_step": ([P, P, P, P, P, I, I, I, I, I, I64, P, I64, I, F, P, P, P, SZ, P], I),
        "hata_decode_step_qk": ([P, P, P, P, P, P, I, I, I, I, I, I64, P, I64, I, F, P, P, P, SZ, P], I),
        "hata_decode_step_noalloc": ([P, P, P, P, P, I, I, I, I, I, I64, P, I64, I, F, P, P, P], I),
        "hata_dense_decode": ([P, P, P, I, I, I, I, I64, P, I64, F, P, P, SZ, P], I),
        "hata_workspace_bytes": ([I, I, I, I, I, I, I64, I], SZ),
        "hata_workspace_reset": ([P, SZ, P], I),
        "hata_workspace_check": ([P, SZ, ctypes.POINTER(I), P], I),
        "hata_workspace_set_spin_limit": ([P, SZ, ctypes.c_uint32, P], I),
        "hata_stream_read": ([P, SZ, P, SZ, P], I),
        "hata_hash_labels": ([P, P, P, I, I, I, I, F, F, P, P], I),
        "hata_hash_train_step": ([P, P, P, P, I, I, I, I, F, F, F, F, F, P, P, P, P, SZ, P], I),
        "hata_hash_train_workspace_bytes": ([I, I, I, I], SZ),
        "hata_prefill": ([P, P, P, P, P, I, I, I, I, I, I64, I64, P, I64, F, P, P], I),
        "hata_decode_step_paged": ([P, P, P, P, P, P, I, I, I, I, I, I, I, I, P, I64, I, F, P, P, P, SZ, P], I),
        "hata_prefill_paged": ([P, P, P, P, P, P, I, I, I, I, I, I, I, I, I64, P, I64, F, P, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def exported_symbols() -> list[str]:
    return [n for n in ("hata_status_string", "hata_last_error_message", "hata_version",
                        "hata_encode_append", "hata_hamming_scores", "hata_topk",
                        "hata_sparse_decode", "hata_decode_step", "hata_decode_step_qk",
                        "hata_decode_step_noalloc",
                        "hata_dense_decode",
                        "hata_workspace_bytes", "hata_workspace_reset", "hata_workspace_check",
                        "hata_workspace_set_spin_limit",
                        "hata_stream_read", "hata_hash_labels", "hata_hash_train_step",
                        "hata_hash_train_workspace_bytes", "hata_prefill", "hata_decode_step_paged",
                        "hata_prefill_paged")
            if hasattr(load(), n)]


def _check(rc: int) -> None:
    if rc != 0:
        L = load()
        raise HataError(rc, f"{L.hata_status_string(rc).decode()} -- {L.hata_last_error_message().decode()}")


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, dtype: torch.dtype, name: str) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _need_codes(t: torch.Tensor, r: int, name: str) -> None:
    """A code tensor for r-bit codes: int32 rows of r/32 words, or int64 rows
    of r/64 words when r >= 64."""
    if t.dtype == torch.int32:
        ok = t.shape[-1] == r // 32
    elif t.dtype == torch.int64:
        ok = r >= 64 and t.shape[-1] == r // 64
    else:
        raise TypeError(f"{name} must be torch.int32 or torch.int64, got {t.dtype}")
    if not ok:
        raise ValueError(f"{name}: last dimension {t.shape[-1]} ({t.dtype}) does not hold {r}-bit codes")


def code_bits(t: torch.Tensor) -> int:
    """Code width r of a code tensor (from its last dimension and dtype)."""
    return t.shape[-1] * (32 if t.dtype == torch.int32 else 64)


def new_codes(*shape: int, r: int = 128, device="cuda", fill: int = 0) -> torch.Tensor:
    """A code tensor [*shape, words] for r-bit codes: int64 words for r >= 64,
    one int32 word per row at r = 32."""
    if r >= 64:
        return torch.full((*shape, r // 64), fill, dtype=torch.int64, device=device)
    return torch.full((*shape, r // 32), fill, dtype=torch.int32, device=device)


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ----------------------------------------------------------------- entry points

def encode_append(x: torch.Tensor, W_H: torch.Tensor, codes: torch.Tensor, n_new: int,
                  pos: torch.Tensor | None = None, stream=None) -> None:
    """x bf16 [B,H,x_rows,d]; W_H f32 [Hkv,d,r]; codes [B,H,cap,words] holding
    r-bit code rows (r in 32, 64, 128, 256; see `new_codes`)."""
    _need(x, torch.bfloat16, "x")
    _need(W_H, torch.float32, "W_H")
    if pos is not None:
        _need(pos, torch.int32, "pos")
    B, H, x_rows, d = x.shape
    Hkv, _, r = W_H.shape
    _need_codes(codes, r, "codes")
    cap = codes.shape[2]
    _check(load().hata_encode_append(_ptr(x), x_rows, B, H, int(n_new), _ptr(W_H), Hkv, d, r,
                                     _ptr(codes), cap, _ptr(pos), _stream(stream)))


def hamming_scores(q_codes: torch.Tensor, k_codes: torch.Tensor, seq_lens: torch.Tensor,
                   max_len: int, scores: torch.Tensor, stream=None, r: int | None = None) -> None:
    """q_codes [B,Hq,words]; k_codes [B,Hkv,cap,words] (r-bit code rows, see
    `new_codes`); scores int16 [B,Hkv,cap].  r defaults to the width the
    code tensors hold."""
    r = int(r or code_bits(q_codes))
    _need_codes(q_codes, r, "q_codes")
    _need_codes(k_codes, r, "k_codes")
    _need(scores, torch.int16, "scores")
    _need(seq_lens, torch.int32, "seq_lens")
    B, Hq, _ = q_codes.shape
    _, Hkv, cap, _ = k_codes.shape
    _check(load().hata_hamming_scores(_ptr(q_codes), _ptr(k_codes), B, Hq, Hkv, r, cap,
                                      _ptr(seq_lens), int(max_len), _ptr(scores), _stream(stream)))


def topk(scores: torch.Tensor, seq_lens: torch.Tensor, max_len: int, k: int, max_score: int,
         idx: torch.Tensor, stream=None, ws: torch.Tensor | None = None) -> None:
    """scores int16 [B,Hkv,cap]; idx int32 [B,Hkv,k].  ws (uint8, at least
    workspace_bytes(OP_TOPK, ...)) lets long sequences use many workgroups."""
    _need(scores, torch.int16, "scores")
    _need(idx, torch.int32, "idx")
    _need(seq_lens, torch.int32, "seq_lens")
    B, Hkv, cap = scores.shape
    _check(load().hata_topk(_ptr(scores), B, Hkv, cap, _ptr(seq_lens), int(max_len), int(k),
                            int(max_score), _ptr(idx), _ptr(ws), 0 if ws is None else ws.numel(),
                            _stream(stream)))


def workspace_bytes(op: int, B: int, Hq: int, Hkv: int, max_len: int, k: int, d: int = 128,
                    r: int = 128) -> int:
    return int(load().hata_workspace_bytes(op, B, Hq, Hkv, d, r, int(max_len), int(k)))


def alloc_workspace(op: int, B: int, Hq: int, Hkv: int, max_len: int, k: int,
                    device="cuda", r: int = 128) -> torch.Tensor:
    """A zeroed workspace tensor (uint8) for operation `op` at these sizes
    (r: code width in bits)."""
    n = max(workspace_bytes(op, B, Hq, Hkv, max_len, k, r=r), 256)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def sparse_decode(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, idx: torch.Tensor,
                  scale: float, out: torch.Tensor, ws: torch.Tensor, stream=None) -> None:
    """q bf16 [B,Hq,d]; K,V bf16 [B,Hkv,cap,d]; idx int32 [B,Hkv,k]; out f32 [B,Hq,d]."""
    for t, n in ((q, "q"), (K, "K"), (V, "V")):
        _need(t, torch.bfloat16, n)
    _need(idx, torch.int32, "idx")
    _need(out, torch.float32, "out")
    B, Hq, d = q.shape
    _, Hkv, cap, _ = K.shape
    k = idx.shape[2]
    _check(load().hata_sparse_decode(_ptr(q), _ptr(K), _ptr(V), B, Hq, Hkv, d, cap, _ptr(idx), k,
                                     float(scale), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))


def dense_decode(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, seq_lens: torch.Tensor,
                 max_len: int, scale: float, out: torch.Tensor, ws: torch.Tensor,
                 stream=None) -> None:
    for t, n in ((q, "q"), (K, "K"), (V, "V")):
        _need(t, torch.bfloat16, n)
    _need(out, torch.float32, "out")
    _need(seq_lens, torch.int32, "seq_lens")
    B, Hq, d = q.shape
    _, Hkv, cap, _ = K.shape
    _check(load().hata_dense_decode(_ptr(q), _ptr(K), _ptr(V), B, Hq, Hkv, d, cap, _ptr(seq_lens),
                                    int(max_len), float(scale), _ptr(out), _ptr(ws), ws.numel(),
                                    _stream(stream)))


def prefill(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, W_H: torch.Tensor, codes: torch.Tensor,
            seq_lens: torch.Tensor, max_len: int, scale: float, out: torch.Tensor, stream=None) -> None:
    """Causal prompt attention with the prompt keys' codes written to the cache.
    q bf16 [B,Hq,q_rows,d]; K,V bf16 [B,Hkv,cap,d]; W_H f32 [Hkv,d,r]; codes int64
    [B,Hkv,cap,words] (r-bit code rows, see `new_codes`); seq_lens int32 [B]; out f32
    [B,Hq,q_rows,d]."""
    for t, n in ((q, "q"), (K, "K"), (V, "V")):
        _need(t, torch.bfloat16, n)
    _need(W_H, torch.float32, "W_H")
    _need_codes(codes, W_H.shape[2], "codes")
    _need(seq_lens, torch.int32, "seq_lens")
    _need(out, torch.float32, "out")
    B, Hq, q_rows, d = q.shape
    _, Hkv, cap, _ = K.shape
    r = W_H.shape[2]
    _check(load().hata_prefill(_ptr(q), _ptr(K), _ptr(V), _ptr(W_H), _ptr(codes), B, Hq, Hkv, d, r, q_rows, cap,
                               _ptr(seq_lens), int(max_len), float(scale), _ptr(out), _stream(stream)))


def decode_step_paged(q: torch.Tensor, K_pool: torch.Tensor, V_pool: torch.Tensor, W_H: torch.Tensor,
                      code_pool: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor, max_len: int,
                      k: int, scale: float, out: torch.Tensor, ws: torch.Tensor, idx_out: torch.Tensor | None = None,
                      stream=None) -> None:
    """q bf16 [B,Hq,d]; K_pool, V_pool bf16 [pages,Hkv,P,d]; code_pool [pages,Hkv,P,words] (code rows, see `new_codes`);
    block_table int32 [B,max_pages]; out f32 [B,Hq,d]; idx_out int32 [B,Hkv,k] or None."""
    for t, n in ((q, "q"), (K_pool, "K_pool"), (V_pool, "V_pool")):
        _need(t, torch.bfloat16, n)
    _need(W_H, torch.float32, "W_H")
    _need_codes(code_pool, W_H.shape[2], "code_pool")
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    _need(out, torch.float32, "out")
    if idx_out is not None:
        _need(idx_out, torch.int32, "idx_out")
    B, Hq, d = q.shape
    num_pages, Hkv, P, _ = K_pool.shape
    r = W_H.shape[2]
    _check(load().hata_decode_step_paged(_ptr(q), _ptr(K_pool), _ptr(V_pool), _ptr(W_H), _ptr(code_pool),
                                         _ptr(block_table), block_table.shape[1], num_pages, P, B, Hq, Hkv, d, r,
                                         _ptr(seq_lens), int(max_len), int(k), float(scale), _ptr(out),
                                         _ptr(idx_out), _ptr(ws), ws.numel(), _stream(stream)))


def prefill_paged(q: torch.Tensor, K_pool: torch.Tensor, V_pool: torch.Tensor, W_H: torch.Tensor,
                  code_pool: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor, max_len: int,
                  scale: float, out: torch.Tensor, stream=None) -> None:
    """hata_prefill into page pools: q bf16 [B,Hq,q_rows,d]; K_pool, V_pool bf16 [pages,Hkv,P,d];
    code_pool [pages,Hkv,P,words] (code rows, see `new_codes`); block_table int32 [B,max_pages]; out f32 [B,Hq,q_rows,d]."""
    for t, n in ((q, "q"), (K_pool, "K_pool"), (V_pool, "V_pool")):
        _need(t, torch.bfloat16, n)
    _need(W_H, torch.float32, "W_H")
    _need_codes(code_pool, W_H.shape[2], "code_pool")
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    _need(out, torch.float32, "out")
    B, Hq, q_rows, d = q.shape
    num_pages, Hkv, P, _ = K_pool.shape
    r = W_H.shape[2]
    _check(load().hata_prefill_paged(_ptr(q), _ptr(K_pool), _ptr(V_pool), _ptr(W_H), _ptr(code_pool),
                                     _ptr(block_table), block_table.shape[1], num_pages, P, B, Hq, Hkv, d, r, q_rows,
                                     _ptr(seq_lens), int(max_len), float(scale), _ptr(out), _stream(stream)))


def stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read all of `src` once (measurement of the HBM read rate); sink int64 [>= 1024]."""
    _need(sink, torch.int64, "sink")
    _check(load().hata_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                   sink.numel(), _stream(stream)))


def decode_step(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, W_H: torch.Tensor,
                codes: torch.Tensor, seq_lens: torch.Tensor, max_len: int, k: int, scale: float,
                out: torch.Tensor, ws: torch.Tensor, idx_out: torch.Tensor | None = None,
                stream=None) -> None:
    """The fused decode step (see hata_decode_step)."""
    for t, n in ((q, "q"), (K, "K"), (V, "V")):
        _need(t, torch.bfloat16, n)
    _need(W_H, torch.float32, "W_H")
    _need_codes(codes, W_H.shape[2], "codes")
    _need(out, torch.float32, "out")
    _need(seq_lens, torch.int32, "seq_lens")
    if idx_out is not None:
        _need(idx_out, torch.int32, "idx_out")
    B, Hq, d = q.shape
    _, Hkv, cap, _ = K.shape
    r = W_H.shape[2]
    _check(load().hata_decode_step(_ptr(q), _ptr(K), _ptr(V), _ptr(W_H), _ptr(codes), B, Hq, Hkv,
                                   d, r, cap, _ptr(seq_lens), int(max_len), int(k), float(scale),
                                   _ptr(out), _ptr(idx_out), _ptr(ws), ws.numel(), _stream(stream)))


def decode_step_noalloc(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, W_H: torch.Tensor,
                        codes: torch.Tensor, seq_lens: torch.Tensor, max_len: int, k: int, scale: float,
                        out: torch.Tensor, idx_out: torch.Tensor | None = None, stream=None) -> None:
    """The fused decode step without a workspace argument (see
    hata_decode_step_noalloc: the library's static scratch serves)."""
    for t, n in ((q, "q"), (K, "K"), (V, "V")):
        _need(t, torch.bfloat16, n)
    _need(W_H, torch.float32, "W_H")
    _need_codes(codes, W_H.shape[2], "codes")
    _need(out, torch.float32, "out")
    _need(seq_lens, torch.int32, "seq_lens")
    if idx_out is not None:
        _need(idx_out, torch.int32, "idx_out")
    B, Hq, d = q.shape
    _, Hkv, cap, _ = K.shape
    r = W_H.shape[2]
    _check(load().hata_decode_step_noalloc(_ptr(q), _ptr(K), _ptr(V), _ptr(W_H), _ptr(codes), B, Hq, Hkv,
                                           d, r, cap, _ptr(seq_lens), int(max_len), int(k), float(scale),
                                           _ptr(out), _ptr(idx_out), _stream(stream)))


def decode_step_qk(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, W_Hq: torch.Tensor,
                   W_Hk: torch.Tensor, codes: torch.Tensor, seq_lens: torch.Tensor, max_len: int, k: int,
                   scale: float, out: torch.Tensor, ws: torch.Tensor, idx_out: torch.Tensor | None = None,
                   stream=None) -> None:
    """The fused decode step with separate query and key encoders (see
    hata_decode_step_qk)."""
    for t, n in ((q, "q"), (K, "K"), (V, "V")):
        _need(t, torch.bfloat16, n)
    _need(W_Hq, torch.float32, "W_Hq")
    _need(W_Hk, torch.float32, "W_Hk")
    _need_codes(codes, W_Hq.shape[2], "codes")
    _need(out, torch.float32, "out")
    _need(seq_lens, torch.int32, "seq_lens")
    if idx_out is not None:
        _need(idx_out, torch.int32, "idx_out")
    B, Hq, d = q.shape
    _, Hkv, cap, _ = K.shape
    r = W_Hq.shape[2]
    _check(load().hata_decode_step_qk(_ptr(q), _ptr(K), _ptr(V), _ptr(W_Hq), _ptr(W_Hk), _ptr(codes), B, Hq,
                                      Hkv, d, r, cap, _ptr(seq_lens), int(max_len), int(k), float(scale),
                                      _ptr(out), _ptr(idx_out), _ptr(ws), ws.numel(), _stream(stream)))


def hash_labels(q: torch.Tensor, k: torch.Tensor, q_pos: torch.Tensor, labels: torch.Tensor,
                pos_permille: int = 100, s_max: float = 20.0, s_min: float = 1.0, stream=None) -> None:
    """q bf16 [J,d]; k bf16 [n,d]; q_pos int32 [J]; labels f32 [J,n] (see hata_hash_labels)."""
    _need(q, torch.bfloat16, "q")
    _need(k, torch.bfloat16, "k")
    _need(q_pos, torch.int32, "q_pos")
    _need(labels, torch.float32, "labels")
    J, d = q.shape
    n = k.shape[0]
    _check(load().hata_hash_labels(_ptr(q), _ptr(k), _ptr(q_pos), J, n, d, int(pos_permille), float(s_max),
                                   float(s_min), _ptr(labels), _stream(stream)))


def hash_train_workspace(J: int, n: int, r: int, d: int = 128, device="cuda") -> torch.Tensor:
    nb = int(load().hata_hash_train_workspace_bytes(J, n, d, r))
    return torch.empty(max(nb, 256), dtype=torch.uint8, device=device)


def hash_train_step(q: torch.Tensor, k: torch.Tensor, q_pos: torch.Tensor, labels: torch.Tensor,
                    W: torch.Tensor, sigma: float, eps: float, eta: float, lam: float, lr: float,
                    loss: torch.Tensor, ws: torch.Tensor, grad: torch.Tensor | None = None,
                    stream=None) -> None:
    """One gradient step on W f32 [d,r] in place (see hata_hash_train_step); loss f32 [4]."""
    _need(q, torch.bfloat16, "q")
    _need(k, torch.bfloat16, "k")
    _need(q_pos, torch.int32, "q_pos")
    _need(labels, torch.float32, "labels")
    _need(W, torch.float32, "W")
    _need(loss, torch.float32, "loss")
    if grad is not None:
        _need(grad, torch.float32, "grad")
    J, d = q.shape
    n = k.shape[0]
    r = W.shape[1]
    _check(load().hata_hash_train_step(_ptr(q), _ptr(k), _ptr(q_pos), _ptr(labels), J, n, d, r, float(sigma),
                                       float(eps), float(eta), float(lam), float(lr), _ptr(W), _ptr(grad),
                                       _ptr(loss), _ptr(ws), ws.numel(), _stream(stream)))


def workspace_reset(ws: torch.Tensor, stream=None) -> None:
    _check(load().hata_workspace_reset(_ptr(ws), ws.numel(), _stream(stream)))


def workspace_set_spin_limit(ws: torch.Tensor, polls: int, stream=None) -> None:
    _check(load().hata_workspace_set_spin_limit(_ptr(ws), ws.numel(), int(polls), _stream(stream)))


def workspace_check(ws: torch.Tensor, stream=None) -> int:
    err = ctypes.c_int(0)
    _check(load().hata_workspace_check(_ptr(ws), ws.numel(), ctypes.byref(err), _stream(stream)))
    return err.value


def status_string(status: int) -> str:
    return load().hata_status_string(int(status)).decode()


def raw_call(name: str, *args) -> int:
    """Call a C entry point with raw ctypes arguments (tests of the error paths)."""
    return int(getattr(load(), name)(*args))


def last_error_message() -> str:
    return load().hata_last_error_message().decode()
