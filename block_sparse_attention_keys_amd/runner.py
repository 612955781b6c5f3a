"""Device-side driver of a workload through the C ABI.

Marshalling only: allocates the caches in the layouts of ``include/qsa.h``,
copies a workload's cached context into them, builds the pooled indexer
cache with the library's own ``qsa_pool_keys`` kernel, uploads the per-call
inputs, and calls ``qsa_forward``.  No step of the method is computed here.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np
import torch

from . import qsa
from .workloads import BF16, Case, kv_scales


def _dev(a: np.ndarray, device, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(device, non_blocking=False)


def _round(x: int, m: int) -> int:
    return (x + m - 1) // m * m


class DeviceCase:
    """Caches + per-call inputs of one workload on one GPU.

    n_layers independent copies of the caches can be made (the same values
    in distinct buffers), so that a benchmark can rotate over layers the way
    a model does and no step re-reads another step's data from cache memory.
    page_offset places a paged cache's pages above that many unused pages.
    """

    def __init__(self, case: Case, device="cuda", n_layers: int = 1, extra_steps: int = 0,
                 layout: Optional[str] = None, attn_scale: float = 0.0,
                 idx_scale: float = 0.0, budget: Optional[int] = None,
                 block_size: Optional[int] = None, page_offset: int = 0,
                 kv_fp8: Optional[bool] = None, kv_rotate: Optional[bool] = None,
                 kv_scale: Optional[tuple] = None, idx_rope: tuple = (0, 0.0)):
        sp = case.spec
        self.case, self.spec, self.device = case, sp, torch.device(device)
        self.dt = torch.bfloat16 if sp.dtype == BF16 else torch.float32
        B = sp.n_seqs
        self.B = B
        r = sp.block_size if block_size is None else block_size
        self.r = r
        self.kv8 = sp.kv_fp8 if kv_fp8 is None else kv_fp8
        self.kv_rotate = bool(self.kv8 and (sp.kv_rotate if kv_rotate is None else kv_rotate))
        if not self.kv8:
            kv_scale = (1.0, 1.0)
        elif kv_scale is None:
            kv_scale = kv_scales(sp.head_dim, self.kv_rotate)
        self.k_scale, self.v_scale = (float(x) for x in kv_scale)
        self.params = qsa.make_params(sp.n_q_heads, sp.n_kv_heads, sp.head_dim, sp.n_idx_heads,
                                      sp.idx_dim, r, sp.budget if budget is None else budget,
                                      qsa.QSA_BF16 if sp.dtype == BF16 else qsa.QSA_F32,
                                      attn_scale=attn_scale, idx_scale=idx_scale,
                                      kv_dtype=qsa.QSA_KV_FP8 if self.kv8 else qsa.QSA_KV_SAME,
                                      kv_rotate=int(self.kv_rotate), k_scale=self.k_scale,
                                      v_scale=self.v_scale, idx_rope_dim=idx_rope[0],
                                      idx_rope_theta=idx_rope[1])
        self.n_tok = [int(x.shape[0]) for x in case.k]
        cap_tok = max(self.n_tok) + extra_steps
        self.paged = (layout or ("paged" if sp.page_size else "contiguous")) == "paged"
        self.page_size = sp.page_size if sp.page_size else 64
        Hkv, D, dI = sp.n_kv_heads, sp.head_dim, sp.idx_dim
        if self.paged:
            ps = self.page_size
            self.cap = _round(cap_tok, ps)
            self.max_pages = self.cap // ps
            if case.page_table is not None and extra_steps == 0 and layout is None and not page_offset:
                pt = case.page_table.copy()
                n_pages = case.n_pages
            else:  # build a permuted page table with room for the extra steps
                need = [(_round(n + extra_steps, ps)) // ps for n in self.n_tok]
                n_pages = int(sum(need))
                perm = np.random.default_rng(1234).permutation(n_pages).astype(np.int32)
                pt = np.full((B, self.max_pages), -1, np.int32)
                o = 0
                for b in range(B):
                    pt[b, :need[b]] = perm[o:o + need[b]]
                    o += need[b]
            if pt.shape[1] < self.max_pages:
                pt = np.concatenate([pt, np.full((B, self.max_pages - pt.shape[1]), -1, np.int32)], 1)
            if page_offset:  # the sequences' pages at the top of a larger pool
                pt = np.where(pt >= 0, pt + page_offset, pt).astype(np.int32)
                n_pages += page_offset
            self.n_pages = int(n_pages)
            self.page_table_np = pt
            self.page_table = torch.from_numpy(pt).to(self.device)
            kv_shape = (self.n_pages, Hkv, ps, D)
            ki_shape = (self.n_pages, ps, dI)
        else:
            self.cap = _round(cap_tok, 64)
            self.max_pages = 0
            self.n_pages = 0
            self.page_table = None
            kv_shape = (B, Hkv, self.cap, D)
            ki_shape = (B, self.cap, dI)
        self.layers: List[dict] = []
        base = self._alloc(kv_shape, ki_shape)
        self._fill_context(base)
        self.layers.append(base)
        for _ in range(1, n_layers):
            cp = {k: v.clone() for k, v in base.items()}
            self.layers.append(cp)
        torch.cuda.synchronize(self.device)

    # ------------------------------------------------------------------ setup
    def _alloc(self, kv_shape, ki_shape) -> dict:
        sp = self.spec
        kv_dt = torch.uint8 if self.kv8 else self.dt
        st = {"k": torch.zeros(kv_shape, dtype=kv_dt, device=self.device),
              "v": torch.zeros(kv_shape, dtype=kv_dt, device=self.device)}
        if self.r > 0:
            st["kI"] = torch.zeros(ki_shape, dtype=self.dt, device=self.device)
            b0 = self.batch_for([0] * self.B, [1] * self.B)
            ld = qsa.qsa_pooled_ld(self.params, b0)
            self.pooled_ld = ld
            st["pooled"] = torch.zeros((self.B, sp.idx_dim, ld), dtype=torch.float32,
                                       device=self.device)
        return st

    def cached_rows(self, which: str, b: int, n: int, layer: int = 0) -> torch.Tensor:
        """Rows [0, n) of sequence b of cache `which` ("k" or "v") as [n][Hkv][D]."""
        st = self.layers[layer][which]
        s = torch.arange(n, device=self.device)
        if self.paged:
            pg, off = self._rows(b, s)
            return st[pg, :, off, :]
        return st[b, :, :n, :].permute(1, 0, 2)

    def _rows(self, b: int, s: torch.Tensor):
        """Cache coordinates of token positions s of sequence b."""
        if self.paged:
            pt = self.page_table[b]
            return pt[s // self.page_size].long(), (s % self.page_size).long()
        return None, s

    def _fill_context(self, st: dict) -> None:
        """Copy each sequence's cached context rows into the caches (8-bit
        caches: stored by the library's qsa_store_kv, one sequence at a
        time), then pool the context's indexer keys with the library kernel."""
        case = self.case
        ctx = case.ctx
        for b in range(self.B):
            n = ctx[b]
            if n == 0:
                continue
            s = torch.arange(n, device=self.device)
            kk = _dev(case.k[b][:n], self.device, self.spec.dtype)
            vv = _dev(case.v[b][:n], self.device, self.spec.dtype)
            if self.kv8:
                counts = [0] * self.B
                counts[b] = n
                qsa.qsa_store_kv(self.params, self.batch_for([0] * self.B, counts), kk, vv,
                                 st["k"], st["v"])
                torch.cuda.synchronize(self.device)
            elif self.paged:
                pg, off = self._rows(b, s)
                st["k"][pg, :, off, :] = kk
                st["v"][pg, :, off, :] = vv
            else:
                st["k"][b, :, :n, :] = kk.permute(1, 0, 2)
                st["v"][b, :, :n, :] = vv.permute(1, 0, 2)
            del kk, vv
        if self.r > 0 and sum(ctx) > 0:
            kI_new = torch.cat([_dev(case.kI[b][:ctx[b]], self.device, self.spec.dtype)
                                for b in range(self.B)])
            batch = self.batch_for([0] * self.B, list(ctx))
            ws = None
            qsa.qsa_pool_keys(self.params, batch, kI_new, st["kI"], st["pooled"])
            torch.cuda.synchronize(self.device)
            del kI_new

    # ------------------------------------------------------------------ calls
    def batch_for(self, past: List[int], n_new: List[int]) -> qsa.Batch:
        cu = np.zeros(self.B + 1, np.int32)
        cu[1:] = np.cumsum(n_new)
        cu_t = torch.from_numpy(cu).to(self.device)
        past_t = torch.from_numpy(np.asarray(past, np.int32)).to(self.device)
        T = int(cu[-1])
        return qsa.Batch(self.B, T, max(1, max(n_new)), max(p + n for p, n in zip(past, n_new)),
                         self.cap, cu_t, past_t, self.page_table,
                         self.page_size if self.paged else 0, self.max_pages, self.n_pages)

    def call_inputs(self, i: int) -> dict:
        """Device inputs of call i of the workload (positions [start, end) per sequence)."""
        case = self.case
        spans = case.calls[i]
        past = [s for s, _ in spans]
        n_new = [e - s for s, e in spans]
        cat = lambda xs: np.concatenate(xs, axis=0)  # noqa: E731
        qi = [(s - int(case.q_pos[b][0]), e - int(case.q_pos[b][0])) for b, (s, e) in enumerate(spans)]
        host = {
            "k_new": cat([case.k[b][s:e] for b, (s, e) in enumerate(spans)]),
            "v_new": cat([case.v[b][s:e] for b, (s, e) in enumerate(spans)]),
            "kI_new": cat([case.kI[b][s:e] for b, (s, e) in enumerate(spans)]),
            "q": cat([case.q[b][a:c] for b, (a, c) in enumerate(qi)]),
            "qI": cat([case.qI[b][a:c] for b, (a, c) in enumerate(qi)]),
            "w": cat([case.w[b][a:c] for b, (a, c) in enumerate(qi)]),
            "gate": cat([case.gate[b][a:c] for b, (a, c) in enumerate(qi)]),
        }
        d = {k: _dev(v, self.device, self.spec.dtype) for k, v in host.items()}
        d["batch"] = self.batch_for(past, n_new)
        d["T"] = int(sum(n_new))
        d["spans"] = spans
        return d

    def alloc_outputs(self, inp: dict) -> dict:
        sp = self.spec
        T = inp["T"]
        k = max(1, (self.params.budget // self.r) if self.r else 1)
        ws_bytes = qsa.qsa_workspace_size(self.params, inp["batch"])
        return {"out": torch.empty((T, sp.n_q_heads, sp.head_dim), dtype=self.dt, device=self.device),
                "sel": torch.empty((T, k), dtype=torch.int32, device=self.device),
                "n_blocks": torch.empty((T,), dtype=torch.int32, device=self.device),
                "ws": torch.zeros((max(ws_bytes, 16),), dtype=torch.uint8, device=self.device)}

    def forward(self, inp: dict, outs: dict, layer: int = 0, stream=None) -> None:
        st = self.layers[layer]
        qsa.qsa_forward(self.params, inp["batch"], inp["q"], inp["k_new"], inp["v_new"],
                        inp["qI"], inp["kI_new"], inp["w"], inp["gate"], st["k"], st["v"],
                        st.get("kI"), st.get("pooled"), outs["out"], outs["sel"],
                        outs["n_blocks"], outs["ws"], stream)


class BlockDeviceCase:
    """Caches (empty at first), weights and per-call inputs of a QSA block
    workload on one GPU; every call goes through qsa_block_forward.  The
    context is filled by the block's own prefill calls."""

    def __init__(self, bc, device="cuda", layout: str = "paged", page_size: int = 64,
                 kv_fp8: bool = False, kv_rotate: bool = False):
        sp = bc.spec
        self.bc, self.spec, self.device = bc, sp, torch.device(device)
        B = sp.n_seqs
        self.B, self.r = B, sp.block_size
        self.kv8, self.kv_rotate = kv_fp8, bool(kv_fp8 and kv_rotate)
        # (the block's k and v are RMS-normed / unit-variance: the rotated
        # values' scale follows as for the workload draws, times sqrt(D))
        sd = (1.0 if self.kv_rotate else sp.head_dim ** -0.5) * sp.head_dim ** 0.5
        self.k_scale = self.v_scale = float(np.float32(8.0 * sd / 448.0)) if kv_fp8 else 1.0
        self.params = qsa.make_params(sp.n_q_heads, sp.n_kv_heads, sp.head_dim, sp.n_idx_heads,
                                      sp.idx_dim, sp.block_size, sp.budget, qsa.QSA_BF16,
                                      idx_rope_dim=bc.idx_rope_dim,
                                      idx_rope_theta=bc.idx_rope_theta,
                                      kv_dtype=qsa.QSA_KV_FP8 if kv_fp8 else qsa.QSA_KV_SAME,
                                      kv_rotate=int(self.kv_rotate), k_scale=self.k_scale,
                                      v_scale=self.v_scale)
        self.block = qsa.make_block_params(bc.d_model, bc.rotary_dim, bc.rope_theta, bc.norm_eps)
        Hkv, D, dI = sp.n_kv_heads, sp.head_dim, sp.idx_dim
        n_tok = bc.n_tok
        self.paged = layout == "paged"
        self.page_size = page_size
        if self.paged:
            ps = page_size
            need = [_round(n, ps) // ps for n in n_tok]
            self.max_pages = max(need)
            self.cap = self.max_pages * ps
            self.n_pages = int(sum(need))
            perm = np.random.default_rng(4321).permutation(self.n_pages).astype(np.int32)
            pt = np.full((B, self.max_pages), -1, np.int32)
            o = 0
            for b in range(B):
                pt[b, :need[b]] = perm[o:o + need[b]]
                o += need[b]
            self.page_table = torch.from_numpy(pt).to(self.device)
            kv_shape, ki_shape = (self.n_pages, Hkv, ps, D), (self.n_pages, ps, dI)
        else:
            self.cap = _round(max(n_tok), 64)
            self.max_pages = self.n_pages = 0
            self.page_table = None
            kv_shape, ki_shape = (B, Hkv, self.cap, D), (B, self.cap, dI)
        bf = torch.bfloat16
        kv_dt = torch.uint8 if kv_fp8 else bf
        self.st = {"k": torch.zeros(kv_shape, dtype=kv_dt, device=self.device),
                   "v": torch.zeros(kv_shape, dtype=kv_dt, device=self.device)}
        if self.r > 0:
            self.st["kI"] = torch.zeros(ki_shape, dtype=bf, device=self.device)
            ld = qsa.qsa_pooled_ld(self.params, self.batch_for([0] * B, [1] * B))
            self.st["pooled"] = torch.zeros((B, dI, ld), dtype=torch.float32, device=self.device)
        dev = lambda a: _dev(a, self.device, BF16)  # noqa: E731
        self.w_in, self.w_o = dev(bc.w_in), dev(bc.w_o)
        self.q_norm, self.k_norm = dev(bc.q_norm), dev(bc.k_norm)

    def batch_for(self, past: List[int], n_new: List[int]) -> qsa.Batch:
        cu = np.zeros(self.B + 1, np.int32)
        cu[1:] = np.cumsum(n_new)
        T = int(cu[-1])
        return qsa.Batch(self.B, T, max(1, max(n_new)), max(p + n for p, n in zip(past, n_new)),
                         self.cap, torch.from_numpy(cu).to(self.device),
                         torch.from_numpy(np.asarray(past, np.int32)).to(self.device),
                         self.page_table, self.page_size if self.paged else 0, self.max_pages,
                         self.n_pages)

    def call_inputs(self, i: int) -> dict:
        spans = self.bc.calls[i]
        x = np.concatenate([self.bc.x[b][s:e] for b, (s, e) in enumerate(spans)], 0)
        batch = self.batch_for([s for s, _ in spans], [e - s for s, e in spans])
        T = int(x.shape[0])
        k = max(1, self.params.budget // self.r if self.r else 1)
        ws = max(qsa.qsa_block_workspace_size(self.params, self.block, batch), 16)
        return {"x": _dev(x, self.device, BF16), "batch": batch, "T": T, "spans": spans,
                "y": torch.empty((T, self.bc.d_model), dtype=torch.bfloat16, device=self.device),
                "sel": torch.empty((T, k), dtype=torch.int32, device=self.device),
                "n_blocks": torch.empty((T,), dtype=torch.int32, device=self.device),
                "ws": torch.zeros((ws,), dtype=torch.uint8, device=self.device)}

    def forward(self, c: dict, stream=None) -> None:
        st = self.st
        qsa.qsa_block_forward(self.params, self.block, c["batch"], c["x"], self.w_in, self.q_norm,
                              self.k_norm, self.w_o, st["k"], st["v"], st.get("kI"),
                              st.get("pooled"), c["y"], c["sel"], c["n_blocks"], c["ws"], stream)
