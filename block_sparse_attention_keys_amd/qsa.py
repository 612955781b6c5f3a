"""ctypes binding of ``libqsa.so`` (the QSA hot path on gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in ``include/qsa.h``.  Arguments may be torch
tensors (their ``data_ptr()`` is passed), raw integer device addresses, or
None for optional pointers.  ``stream`` defaults to torch's current stream.
A missing library raises immediately: there is no fallback.
"""
from __future__ import annotations

import contextlib
import ctypes as C
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqsa.so")

QSA_OK = 0
QSA_ERR_INVALID = -1
QSA_ERR_UNSUPPORTED = -2
QSA_ERR_WORKSPACE = -3
QSA_ERR_HIP = -4
QSA_F32 = 0
QSA_BF16 = 1
QSA_KV_SAME = 0
QSA_KV_FP8 = 2

EXPORTS = ["qsa_last_error", "qsa_pooled_ld", "qsa_workspace_size", "qsa_pool_keys",
           "qsa_store_kv", "qsa_score_select", "qsa_attend", "qsa_forward",
           "qsa_forward_noalloc", "qsa_block_workspace_size", "qsa_block_forward"]
QSA_NOALLOC_SCRATCH_BYTES = 16 << 20


class qsa_params(C.Structure):
    _fields_ = [("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("n_idx_heads", C.c_int32), ("idx_dim", C.c_int32), ("block_size", C.c_int32),
                ("ratio", C.c_int32), ("budget", C.c_int32), ("attn_scale", C.c_float),
                ("idx_scale", C.c_float), ("dtype", C.c_int32), ("kv_dtype", C.c_int32),
                ("kv_rotate", C.c_int32), ("k_scale", C.c_float), ("v_scale", C.c_float),
                ("idx_rope_dim", C.c_int32), ("idx_rope_theta", C.c_float)]


class qsa_block_params(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("rotary_dim", C.c_int32), ("rope_theta", C.c_float),
                ("norm_eps", C.c_float)]


class qsa_batch(C.Structure):
    _fields_ = [("n_seqs", C.c_int32), ("n_tokens", C.c_int32), ("max_q_len", C.c_int32),
                ("max_kv_len", C.c_int32), ("kv_capacity", C.c_int32), ("page_size", C.c_int32),
                ("max_pages", C.c_int32), ("n_pages", C.c_int32), ("cu_q", C.c_void_p),
                ("past_len", C.c_void_p), ("page_table", C.c_void_p)]


class QsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"QSA status {status}: {msg}")
        self.status = status


_lib: Optional[C.CDLL] = None


def lib(path: str = LIB_PATH) -> C.CDLL:
    """Load libqsa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = _load(path)
    return _lib


def _load(path: str) -> C.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m block_sparse_attention_keys_amd.build`")
    L = C.CDLL(path)
    P, B = C.POINTER(qsa_params), C.POINTER(qsa_batch)
    vp = C.c_void_p
    L.qsa_last_error.restype = C.c_char_p
    L.qsa_last_error.argtypes = []
    L.qsa_pooled_ld.restype = C.c_int64
    L.qsa_pooled_ld.argtypes = [P, B]
    L.qsa_workspace_size.restype = C.c_size_t
    L.qsa_workspace_size.argtypes = [P, B]
    L.qsa_pool_keys.restype = C.c_int
    L.qsa_pool_keys.argtypes = [P, B, vp, vp, vp, vp]
    L.qsa_store_kv.restype = C.c_int
    L.qsa_store_kv.argtypes = [P, B, vp, vp, vp, vp, vp]
    L.qsa_score_select.restype = C.c_int
    L.qsa_score_select.argtypes = [P, B, vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp]
    L.qsa_attend.restype = C.c_int
    L.qsa_attend.argtypes = [P, B, vp, vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp]
    L.qsa_forward.restype = C.c_int
    L.qsa_forward.argtypes = [P, B] + [vp] * 15 + [C.c_size_t, vp]
    L.qsa_forward_noalloc.restype = C.c_int
    L.qsa_forward_noalloc.argtypes = [P, B] + [vp] * 15
    BP = C.POINTER(qsa_block_params)
    L.qsa_block_workspace_size.restype = C.c_size_t
    L.qsa_block_workspace_size.argtypes = [P, BP, B]
    L.qsa_block_forward.restype = C.c_int
    L.qsa_block_forward.argtypes = [P, BP, B] + [vp] * 13 + [C.c_size_t, vp]
    if hasattr(L, "qsa_probe_keys_visited"):
        L.qsa_probe_keys_visited.restype = C.c_int64
        L.qsa_probe_keys_visited.argtypes = [C.c_int32]
    if hasattr(L, "qsa_probe_library_gemm"):
        L.qsa_probe_library_gemm.restype = None
        L.qsa_probe_library_gemm.argtypes = [C.c_int32]
    if hasattr(L, "qsa_probe_gemm"):
        L.qsa_probe_gemm.restype = C.c_int32
        L.qsa_probe_gemm.argtypes = [vp, vp, vp, C.c_int32, C.c_int32, C.c_int32, C.c_int32, vp]
    return L


PROBE_PATH = os.path.join(PKG, "libqsa_probe.so")


@contextlib.contextmanager
def probe_library(path: str = PROBE_PATH):
    """Route every call of this module through the debug build (include/
    qsa_probe.h) for the duration of the block; yields the loaded library,
    whose qsa_probe_keys_visited reads the rows-loaded counter."""
    global _lib
    saved = _lib
    P = _load(path)
    _lib = P
    try:
        yield P
    finally:
        _lib = saved


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _nbytes(x) -> int:
    if x is None:
        return 0
    return x.numel() * x.element_size()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int) -> None:
    if status != QSA_OK:
        raise QsaError(status, lib().qsa_last_error().decode())


def last_error() -> str:
    return lib().qsa_last_error().decode()


def make_params(n_q_heads, n_kv_heads, head_dim, n_idx_heads, idx_dim, block_size, budget,
                dtype, ratio=None, attn_scale=0.0, idx_scale=0.0, kv_dtype=QSA_KV_SAME,
                kv_rotate=0, k_scale=1.0, v_scale=1.0, idx_rope_dim=0,
                idx_rope_theta=0.0) -> qsa_params:
    return qsa_params(n_q_heads, n_kv_heads, head_dim, n_idx_heads, idx_dim, block_size,
                      block_size if ratio is None else ratio, budget, attn_scale, idx_scale,
                      dtype, kv_dtype, kv_rotate, k_scale, v_scale, idx_rope_dim,
                      idx_rope_theta)


class Batch:
    """A qsa_batch plus the device tensors it points at (kept alive here)."""

    def __init__(self, n_seqs, n_tokens, max_q_len, max_kv_len, kv_capacity, cu_q, past_len,
                 page_table=None, page_size=0, max_pages=0, n_pages=0):
        self.tensors = (cu_q, past_len, page_table)
        self.c = qsa_batch(n_seqs, n_tokens, max_q_len, max_kv_len, kv_capacity, page_size,
                           max_pages, n_pages, _ptr(cu_q), _ptr(past_len), _ptr(page_table))


def _b(batch):
    return batch.c if isinstance(batch, Batch) else batch


def qsa_pooled_ld(params: qsa_params, batch) -> int:
    return int(lib().qsa_pooled_ld(C.byref(params), C.byref(_b(batch))))


def qsa_workspace_size(params: qsa_params, batch) -> int:
    return int(lib().qsa_workspace_size(C.byref(params), C.byref(_b(batch))))


def qsa_pool_keys(params, batch, k_idx_new, k_idx_cache, pooled, stream=None) -> None:
    _check(lib().qsa_pool_keys(C.byref(params), C.byref(_b(batch)), _ptr(k_idx_new),
                               _ptr(k_idx_cache), _ptr(pooled), _stream(stream)))


def qsa_store_kv(params, batch, k_new, v_new, k_cache, v_cache, stream=None) -> None:
    _check(lib().qsa_store_kv(C.byref(params), C.byref(_b(batch)), _ptr(k_new), _ptr(v_new),
                              _ptr(k_cache), _ptr(v_cache), _stream(stream)))


def qsa_score_select(params, batch, q_idx, w, pooled, sel, n_blocks, scores=None, ws=None,
                     stream=None) -> None:
    _check(lib().qsa_score_select(C.byref(params), C.byref(_b(batch)), _ptr(q_idx), _ptr(w),
                                  _ptr(pooled), _ptr(sel), _ptr(n_blocks), _ptr(scores),
                                  _ptr(ws), _nbytes(ws), _stream(stream)))


def qsa_attend(params, batch, q, k_cache, v_cache, sel, n_blocks, gate, out, ws=None,
               stream=None) -> None:
    _check(lib().qsa_attend(C.byref(params), C.byref(_b(batch)), _ptr(q), _ptr(k_cache),
                            _ptr(v_cache), _ptr(sel), _ptr(n_blocks), _ptr(gate), _ptr(out),
                            _ptr(ws), _nbytes(ws), _stream(stream)))


def qsa_forward(params, batch, q, k_new, v_new, q_idx, k_idx_new, w, gate, k_cache, v_cache,
                k_idx_cache, pooled, out, sel=None, n_blocks=None, ws=None,
                stream=None) -> None:
    _check(lib().qsa_forward(C.byref(params), C.byref(_b(batch)), _ptr(q), _ptr(k_new),
                             _ptr(v_new), _ptr(q_idx), _ptr(k_idx_new), _ptr(w), _ptr(gate),
                             _ptr(k_cache), _ptr(v_cache), _ptr(k_idx_cache), _ptr(pooled),
                             _ptr(out), _ptr(sel), _ptr(n_blocks), _ptr(ws), _nbytes(ws),
                             _stream(stream)))


def qsa_forward_noalloc(params, batch, q, k_new, v_new, q_idx, k_idx_new, w, gate, k_cache,
                        v_cache, k_idx_cache, pooled, out, sel=None, n_blocks=None,
                        stream=None) -> None:
    _check(lib().qsa_forward_noalloc(C.byref(params), C.byref(_b(batch)), _ptr(q), _ptr(k_new),
                                     _ptr(v_new), _ptr(q_idx), _ptr(k_idx_new), _ptr(w),
                                     _ptr(gate), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(k_idx_cache), _ptr(pooled), _ptr(out), _ptr(sel),
                                     _ptr(n_blocks), _stream(stream)))


def make_block_params(d_model, rotary_dim, rope_theta, norm_eps=1e-6) -> qsa_block_params:
    return qsa_block_params(d_model, rotary_dim, rope_theta, norm_eps)


def qsa_block_workspace_size(params: qsa_params, block: qsa_block_params, batch) -> int:
    return int(lib().qsa_block_workspace_size(C.byref(params), C.byref(block),
                                              C.byref(_b(batch))))


def qsa_block_forward(params, block, batch, x, w_in, q_norm, k_norm, w_o, k_cache, v_cache,
                      k_idx_cache, pooled, y, sel=None, n_blocks=None, ws=None,
                      stream=None) -> None:
    _check(lib().qsa_block_forward(C.byref(params), C.byref(block), C.byref(_b(batch)), _ptr(x),
                                   _ptr(w_in), _ptr(q_norm), _ptr(k_norm), _ptr(w_o),
                                   _ptr(k_cache), _ptr(v_cache), _ptr(k_idx_cache), _ptr(pooled),
                                   _ptr(y), _ptr(sel), _ptr(n_blocks), _ptr(ws), _nbytes(ws),
                                   _stream(stream)))
