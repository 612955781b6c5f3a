"""Runs a workload through the C ABI on the GPU and compares it with the
CPU oracle on the same seeded inputs (helpers for the GPU parity tests)."""
from __future__ import annotations

import sys
from typing import Dict, List, Optional

import numpy as np
import torch

import oracle
import parity
from block_sparse_attention_keys_amd import qsa, runner, workloads


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dims_of(dc: runner.DeviceCase) -> dict:
    p = dc.params
    return dict(n_q_heads=p.n_q_heads, n_kv_heads=p.n_kv_heads, head_dim=p.head_dim,
                n_idx_heads=p.n_idx_heads, idx_dim=p.idx_dim, block_size=p.block_size,
                budget=p.budget, attn_scale=p.attn_scale, idx_scale=p.idx_scale,
                idx_rope_dim=p.idx_rope_dim, idx_rope_theta=p.idx_rope_theta)


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


class SeqF32:
    """fp32 host views of a sequence's K, V, k_I (converted once)."""

    def __init__(self, case: workloads.Case):
        self.case = case
        self.cache: Dict[int, tuple] = {}

    def get(self, b):
        if b not in self.cache:
            c = self.case
            self.cache[b] = (workloads.as_f32(c.k[b]), workloads.as_f32(c.v[b]),
                             workloads.as_f32(c.kI[b]))
        return self.cache[b]

    def codes(self, b, dc, orc=None):
        """The oracle's 8-bit storage codes of sequence b's K and V under
        dc's storage (rotation, scales)."""
        key = ("codes", b, dc.kv_rotate, dc.k_scale, dc.v_scale)
        if key not in self.cache:
            orc = orc or oracle.load()
            K, V, _ = self.get(b)
            inv_k = float(np.float32(1.0) / np.float32(dc.k_scale))
            inv_v = float(np.float32(1.0) / np.float32(dc.v_scale))
            self.cache[key] = (orc.kv8_encode(K, dc.kv_rotate, inv_k),
                               orc.kv8_encode(V, dc.kv_rotate, inv_v))
        return self.cache[key]


def run_calls(dc: runner.DeviceCase, calls: Optional[List[int]] = None, keep=None):
    """Run calls in order; return per kept call (out, sel, n_blocks, spans)."""
    n = len(dc.case.calls)
    calls = list(range(n)) if calls is None else calls
    res = {}
    for i in calls:
        inp = dc.call_inputs(i)
        outs = dc.alloc_outputs(inp)
        say(f"  gpu call {i}/{n}: T={inp['T']}")
        dc.forward(inp, outs)
        torch.cuda.synchronize()
        if keep is None or i in keep:
            res[i] = (to_np(outs["out"]), outs["sel"].cpu().numpy(),
                      outs["n_blocks"].cpu().numpy(), inp["spans"])
    return res


def kv8_values(orc, codes, rotate: bool, scale: float) -> np.ndarray:
    """fp32 K or V rows that 8-bit codes [..., D] stand for, back in the
    unrotated basis (decode(c) * scale, then H x / D when rotated): the
    input of an oracle attention over a token set the GPU chose."""
    lut = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
    x = lut[np.asarray(codes)] * np.float32(scale)
    if rotate:
        x = orc.fwht(x) / np.float32(x.shape[-1])
    return x.astype(np.float32)


def attend_over_selection(orc, dims, K, V, q, gate, sel_row, n_blocks: int, p: int):
    """The oracle's gated attention of one query at position p over the token
    set of a given selection (blocks sel_row[:n_blocks] plus the tail)."""
    r = dims["block_size"]
    toks = orc.token_set(np.asarray(sel_row[:n_blocks], np.int32), r, p)
    scale = dims["attn_scale"] if dims["attn_scale"] > 0 else dims["head_dim"] ** -0.5
    return orc.attend(q, K, V, gate, toks, scale)


def check_call(dc, seqf: SeqF32, result, sample: Optional[int] = None, rng_seed: int = 0,
               orc=None, max_exempt: int = 0) -> dict:
    """Compare one call's GPU results with the oracle, all queries or a sample
    of them per sequence.  Selections first (bit-exact, or a valid near-tie
    row, at most max_exempt of them: 0 wherever the scores are bit-exact);
    then outputs, a near-tie row's against the oracle's attention over the
    GPU's own selection.  Raises AssertionError on a miss."""
    orc = orc or oracle.load()
    out, sel, nblk, spans = result
    case = dc.case
    dims = dims_of(dc)
    dtype = case.spec.dtype
    kv8 = getattr(dc, "kv8", False)
    rng = np.random.default_rng(rng_seed)
    t0 = 0
    worst = {"max_abs": 0.0, "mean_abs": 0.0, "max_rel": 0.0, "rows": 0, "exempt": 0}
    for b, (s, e) in enumerate(spans):
        n_q = e - s
        if n_q == 0:
            continue  # a sequence with no new tokens in this call: no output rows
        idx = np.arange(n_q)
        if sample is not None and n_q > sample:
            idx = np.sort(rng.choice(n_q, size=sample, replace=False))
        K, V, kI = seqf.get(b)
        qbase = int(case.q_pos[b][0])
        qi = (s - qbase) + idx
        if kv8:
            Kc, Vc = seqf.codes(b, dc, orc)
            ref = orc.sequence_kv8(dims, Kc, Vc, dc.kv_rotate, dc.k_scale, dc.v_scale, kI,
                                   s + idx, case.q[b][qi], case.qI[b][qi], case.w[b][qi],
                                   case.gate[b][qi], want_scores=dims["block_size"] > 0)
        else:
            ref = orc.sequence(dims, K, V, kI, s + idx, case.q[b][qi], case.qI[b][qi],
                               case.w[b][qi], case.gate[b][qi],
                               want_scores=dims["block_size"] > 0)
        ref_out = ref["out"]
        if dims["block_size"] > 0:
            r = dims["block_size"]
            nb = (s + idx + 1) // r
            k = ref["sel"].shape[1]
            got_sel = sel[t0 + idx][:, :k]
            oks, ndiff, ex = parity.selections_ok(got_sel, nblk[t0 + idx], ref["sel"],
                                                  ref["n_blocks"], ref.get("scores"), nb)
            assert oks, f"seq {b}: selections differ in {ndiff} rows"
            worst["exempt"] += len(ex)
            assert worst["exempt"] <= max_exempt, (
                f"seq {b}: {worst['exempt']} near-tie rows (allowed {max_exempt})")
            if ex:
                ref_out = ref_out.copy()
                if kv8:
                    Kx = kv8_values(orc, Kc, dc.kv_rotate, dc.k_scale)
                    Vx = kv8_values(orc, Vc, dc.kv_rotate, dc.v_scale)
                else:
                    Kx, Vx = K, V
                for i in ex:
                    ref_out[i] = attend_over_selection(orc, dims, Kx, Vx, case.q[b][qi[i]],
                                                       case.gate[b][qi[i]], got_sel[i],
                                                       int(ref["n_blocks"][i]), int(s + idx[i]))
        got = out[t0 + idx]
        ok, st = parity.outputs_ok(got, ref_out, dtype)
        assert ok, f"seq {b} outputs {st}"
        for kk in ("max_abs", "mean_abs", "max_rel"):
            worst[kk] = max(worst[kk], st[kk])
        worst["rows"] += len(idx)
        t0 += n_q
    return worst


def pooled_rows(dc: runner.DeviceCase, layer=0) -> np.ndarray:
    """The GPU pooled cache as [B][nb][d_I] (its layout is [B][d_I][ld])."""
    return dc.layers[layer]["pooled"].permute(0, 2, 1).cpu().numpy()
