"""Python access to the QSA CPU oracle (``qsa_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline load this; the product path never does.  It imports nothing from the
HIP package.  Arrays are numpy; bf16 inputs may be passed as raw uint16 bits
and are widened exactly to fp32 here (that widening is the only thing this
wrapper does to values).
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(HERE, "libqsa_oracle.so")


class Dims(C.Structure):
    _fields_ = [("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("n_idx_heads", C.c_int32), ("idx_dim", C.c_int32), ("block_size", C.c_int32),
                ("budget", C.c_int32), ("attn_scale", C.c_float), ("idx_scale", C.c_float),
                ("idx_rope_dim", C.c_int32), ("idx_rope_theta", C.c_float)]


def _f32(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return np.ascontiguousarray((a.astype(np.uint32) << 16).view(np.float32))
    return np.ascontiguousarray(a, dtype=np.float32)


def _p(a: Optional[np.ndarray], t=C.c_float):
    return None if a is None else a.ctypes.data_as(C.POINTER(t))


class Oracle:
    def __init__(self, path: str = DEFAULT_LIB):
        if not os.path.exists(path):
            from . import build as _b  # noqa: F401  (oracle/build.py)
            _b.build(path)
        self.path = path
        L = C.CDLL(path)
        self._L = L
        L.qsa_oracle_threads.restype = C.c_int
        L.qsa_oracle_set_threads.restype = None
        L.qsa_oracle_set_threads.argtypes = [C.c_int]
        L.qsa_oracle_pool.restype = C.c_int64
        L.qsa_oracle_pool.argtypes = [C.POINTER(C.c_float), C.c_int64, C.c_int32, C.c_int32,
                                      C.POINTER(C.c_float)]
        L.qsa_oracle_scores.restype = None
        L.qsa_oracle_scores.argtypes = [C.POINTER(C.c_float), C.POINTER(C.c_float),
                                        C.POINTER(C.c_float), C.c_int64, C.c_int32, C.c_int32,
                                        C.c_float, C.POINTER(C.c_float)]
        L.qsa_oracle_topk.restype = C.c_int32
        L.qsa_oracle_topk.argtypes = [C.POINTER(C.c_float), C.c_int64, C.c_int32,
                                      C.POINTER(C.c_int32)]
        L.qsa_oracle_token_set.restype = C.c_int64
        L.qsa_oracle_token_set.argtypes = [C.POINTER(C.c_int32), C.c_int32, C.c_int32,
                                           C.c_int64, C.POINTER(C.c_int64)]
        L.qsa_oracle_attend.restype = None
        L.qsa_oracle_attend.argtypes = [C.POINTER(C.c_float)] * 4 + [
            C.POINTER(C.c_int64), C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_double,
            C.POINTER(C.c_float)]
        L.qsa_oracle_sequence.restype = C.c_int
        L.qsa_oracle_sequence.argtypes = [
            C.POINTER(Dims), C.c_int64, C.POINTER(C.c_float), C.POINTER(C.c_float),
            C.POINTER(C.c_float), C.c_int64, C.POINTER(C.c_int64), C.POINTER(C.c_float),
            C.POINTER(C.c_float), C.POINTER(C.c_float), C.POINTER(C.c_float),
            C.POINTER(C.c_float), C.POINTER(C.c_int32), C.POINTER(C.c_int32),
            C.POINTER(C.c_int64), C.POINTER(C.c_float), C.c_int64]

        L.qsa_oracle_rope_rows.restype = None
        L.qsa_oracle_rope_rows.argtypes = [C.POINTER(C.c_float), C.c_int64, C.c_int32, C.c_int32,
                                           C.c_double, C.POINTER(C.c_int64)]
        L.qsa_oracle_e4m3_decode.restype = C.c_float
        L.qsa_oracle_e4m3_decode.argtypes = [C.c_uint8]
        L.qsa_oracle_e4m3_encode.restype = C.c_uint8
        L.qsa_oracle_e4m3_encode.argtypes = [C.c_float]
        L.qsa_oracle_fwht.restype = None
        L.qsa_oracle_fwht.argtypes = [C.POINTER(C.c_float), C.c_int32]
        L.qsa_oracle_kv8_encode.restype = None
        L.qsa_oracle_kv8_encode.argtypes = [C.POINTER(C.c_float), C.c_int64, C.c_int32, C.c_int32,
                                            C.c_float, C.POINTER(C.c_uint8)]
        L.qsa_oracle_sequence_kv8.restype = C.c_int
        L.qsa_oracle_sequence_kv8.argtypes = [
            C.POINTER(Dims), C.c_int64, C.POINTER(C.c_uint8), C.POINTER(C.c_uint8), C.c_int32,
            C.c_float, C.c_float, C.POINTER(C.c_float), C.c_int64, C.POINTER(C.c_int64),
            C.POINTER(C.c_float), C.POINTER(C.c_float), C.POINTER(C.c_float),
            C.POINTER(C.c_float), C.POINTER(C.c_float), C.POINTER(C.c_int32),
            C.POINTER(C.c_int32), C.POINTER(C.c_int64), C.POINTER(C.c_float), C.c_int64]

    def threads(self) -> int:
        return int(self._L.qsa_oracle_threads())

    def set_threads(self, n: int) -> None:
        """OpenMP threads of the calling thread's later oracle calls."""
        self._L.qsa_oracle_set_threads(int(n))

    # --- rotary position embedding ---------------------------------------------
    def rope(self, x, R: int, theta: float, pos) -> np.ndarray:
        """qsa_oracle_rope on every row of x [..., n]; pos broadcasts against
        x.shape[:-1] (one position per row)."""
        x = np.array(_f32(x), np.float32, copy=True)
        n = x.shape[-1]
        P = np.ascontiguousarray(np.broadcast_to(np.asarray(pos, np.int64), x.shape[:-1]).reshape(-1))
        flat = x.reshape(-1, n)
        if flat.shape[0]:
            self._L.qsa_oracle_rope_rows(_p(flat), flat.shape[0], n, int(R), float(theta),
                                         _p(P, C.c_int64))
        return x

    # --- 8-bit K/V storage ----------------------------------------------------
    def e4m3_decode(self, codes) -> np.ndarray:
        codes = np.asarray(codes, np.uint8)
        f = self._L.qsa_oracle_e4m3_decode
        return np.array([f(int(c)) for c in codes.ravel()], np.float32).reshape(codes.shape)

    def e4m3_encode(self, x) -> np.ndarray:
        x = np.asarray(x, np.float32)
        f = self._L.qsa_oracle_e4m3_encode
        return np.array([f(float(v)) for v in x.ravel()], np.uint8).reshape(x.shape)

    def fwht(self, x) -> np.ndarray:
        x = np.array(x, np.float32, copy=True)
        n = x.shape[-1]
        flat = np.ascontiguousarray(x.reshape(-1, n))
        for row in flat:
            self._L.qsa_oracle_fwht(_p(row), n)
        return flat.reshape(x.shape)

    def kv8_encode(self, x, rotate: bool, inv_scale: float) -> np.ndarray:
        """Storage codes of rows [..., D] (see qsa_oracle_kv8_encode)."""
        x = _f32(x)
        D = x.shape[-1]
        flat = np.ascontiguousarray(x.reshape(-1, D))
        codes = np.zeros(flat.shape, np.uint8)
        self._L.qsa_oracle_kv8_encode(_p(flat), flat.shape[0], D, int(rotate), inv_scale,
                                      _p(codes, C.c_uint8))
        return codes.reshape(x.shape)

    # --- single steps -------------------------------------------------------
    def pool(self, kI, r: int) -> np.ndarray:
        kI = _f32(kI)
        n, dI = kI.shape
        out = np.zeros((max(n // r, 0), dI), np.float32)
        nb = self._L.qsa_oracle_pool(_p(kI), n, dI, r, _p(out) if out.size else _p(np.zeros(1, np.float32)))
        assert nb == out.shape[0]
        return out

    def scores(self, qI, w, pooled, c: float) -> np.ndarray:
        qI, w, pooled = _f32(qI), _f32(w), _f32(pooled)
        HI, dI = qI.shape
        nb = pooled.shape[0]
        out = np.zeros(max(nb, 1), np.float32)
        self._L.qsa_oracle_scores(_p(qI), _p(w), _p(pooled if nb else np.zeros(1, np.float32)),
                                  nb, HI, dI, c, _p(out))
        return out[:nb]

    def topk(self, s, k: int) -> np.ndarray:
        s = _f32(s)
        sel = np.zeros(max(k, 1), np.int32)
        n = self._L.qsa_oracle_topk(_p(s if s.size else np.zeros(1, np.float32)), s.size, k,
                                    _p(sel, C.c_int32))
        return sel[:n].copy()

    def token_set(self, sel, r: int, p: int) -> np.ndarray:
        sel = np.ascontiguousarray(sel, np.int32)
        cap = len(sel) * max(r, 1) + (p + 1 if r == 0 else r) + 1
        out = np.zeros(cap, np.int64)
        n = self._L.qsa_oracle_token_set(_p(sel if sel.size else np.zeros(1, np.int32), C.c_int32),
                                         len(sel), r, p, _p(out, C.c_int64))
        return out[:n].copy()

    def attend(self, q, K, V, gate, tokens, scale: float) -> np.ndarray:
        q, K, V, gate = _f32(q), _f32(K), _f32(V), _f32(gate)
        tokens = np.ascontiguousarray(tokens, np.int64)
        Hq, D = q.shape
        Hkv = K.shape[1]
        out = np.zeros((Hq, D), np.float32)
        self._L.qsa_oracle_attend(_p(q), _p(K), _p(V), _p(gate), _p(tokens, C.c_int64),
                                  tokens.size, Hq, Hkv, D, scale, _p(out))
        return out

    # --- whole QSA over the queries of one sequence --------------------------
    def sequence_kv8(self, dims: dict, Kc, Vc, rotate: bool, k_scale: float, v_scale: float,
                     kI, pos, q, qI, w, gate, want_scores: bool = False,
                     nb_cap: Optional[int] = None) -> dict:
        """As ``sequence``, with K and V stored as 8-bit codes Kc, Vc
        [n_tok, Hkv, D] (uint8) and scales; see qsa_oracle_sequence_kv8."""
        d = Dims(**{f: dims.get(f, 0) for f, _ in Dims._fields_})
        Kc = np.ascontiguousarray(Kc, np.uint8)
        Vc = np.ascontiguousarray(Vc, np.uint8)
        n_tok = Kc.shape[0]
        kI = _f32(kI) if kI is not None else np.zeros((n_tok, 1), np.float32)
        pos = np.ascontiguousarray(pos, np.int64)
        nq = pos.size
        Hq, D, HI = d.n_q_heads, d.head_dim, max(d.n_idx_heads, 1)
        q, gate = _f32(q).reshape(nq, Hq, D), _f32(gate).reshape(nq, Hq, D)
        qI = _f32(qI).reshape(nq, HI, -1) if qI is not None else np.zeros((nq, 1, 1), np.float32)
        w = _f32(w).reshape(nq, HI) if w is not None else np.zeros((nq, 1), np.float32)
        r = d.block_size
        k = d.budget // r if r > 0 else 0
        out = np.zeros((nq, Hq, D), np.float32)
        sel = np.full((nq, max(k, 1)), -1, np.int32)
        nblk = np.zeros(nq, np.int32)
        ntok = np.zeros(nq, np.int64)
        if nb_cap is None:
            nb_cap = (n_tok // r) if r > 0 else 0
        scores = np.zeros((nq, max(nb_cap, 1)), np.float32) if want_scores else None
        rc = self._L.qsa_oracle_sequence_kv8(
            C.byref(d), n_tok, _p(Kc, C.c_uint8), _p(Vc, C.c_uint8), int(rotate), k_scale,
            v_scale, _p(kI), nq, _p(pos, C.c_int64), _p(q), _p(qI), _p(w), _p(gate), _p(out),
            _p(sel, C.c_int32), _p(nblk, C.c_int32), _p(ntok, C.c_int64), _p(scores), nb_cap)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        res = {"out": out, "sel": sel[:, :k] if k else sel[:, :0], "n_blocks": nblk,
               "n_tokens": ntok}
        if want_scores:
            res["scores"] = scores[:, :nb_cap]
        return res

    def sequence(self, dims: dict, K, V, kI, pos, q, qI, w, gate, want_scores: bool = False,
                 nb_cap: Optional[int] = None) -> dict:
        """QSA outputs of the queries at positions ``pos`` of one sequence.

        K, V [n_tok, Hkv, D]; kI [n_tok, d_I]; q, gate [nq, Hq, D];
        qI [nq, H_I, d_I]; w [nq, H_I].  dims: n_q_heads, n_kv_heads, head_dim,
        n_idx_heads, idx_dim, block_size, budget, attn_scale, idx_scale.
        """
        d = Dims(**{f: dims.get(f, 0) for f, _ in Dims._fields_})
        K, V = _f32(K), _f32(V)
        n_tok = K.shape[0]
        kI = _f32(kI) if kI is not None else np.zeros((n_tok, 1), np.float32)
        pos = np.ascontiguousarray(pos, np.int64)
        nq = pos.size
        Hq, D, HI = d.n_q_heads, d.head_dim, max(d.n_idx_heads, 1)
        q, gate = _f32(q).reshape(nq, Hq, D), _f32(gate).reshape(nq, Hq, D)
        qI = _f32(qI).reshape(nq, HI, -1) if qI is not None else np.zeros((nq, 1, 1), np.float32)
        w = _f32(w).reshape(nq, HI) if w is not None else np.zeros((nq, 1), np.float32)
        r = d.block_size
        k = d.budget // r if r > 0 else 0
        out = np.zeros((nq, Hq, D), np.float32)
        sel = np.full((nq, max(k, 1)), -1, np.int32)
        nblk = np.zeros(nq, np.int32)
        ntok = np.zeros(nq, np.int64)
        if nb_cap is None:
            nb_cap = (n_tok // r) if r > 0 else 0
        scores = np.zeros((nq, max(nb_cap, 1)), np.float32) if want_scores else None
        rc = self._L.qsa_oracle_sequence(
            C.byref(d), n_tok, _p(K), _p(V), _p(kI), nq, _p(pos, C.c_int64), _p(q), _p(qI),
            _p(w), _p(gate), _p(out), _p(sel, C.c_int32), _p(nblk, C.c_int32),
            _p(ntok, C.c_int64), _p(scores), nb_cap)
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        res = {"out": out, "sel": sel[:, :k] if k else sel[:, :0], "n_blocks": nblk,
               "n_tokens": ntok}
        if want_scores:
            res["scores"] = scores[:, :nb_cap]
        return res


_default: Optional[Oracle] = None


def load(path: Optional[str] = None) -> Oracle:
    global _default
    if path is not None:
        return Oracle(path)
    if _default is None:
        _default = Oracle()
    return _default
