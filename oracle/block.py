"""The QSA attention block around the hot path, as the CPU oracle computes it.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): the tests, the smoke
check and the benchmark's CPU baseline use it; the product path never does.

It follows the llama.cpp PR #27739 page, LocalAI QSA-block commit (opening
paragraph): the block is the attention forward end to end -- the q/k/v/o
projections, the q/k norms with the (1 + w) weight polarity, RoPE, the
indexer, the gather consumer, the sigmoid output gate and o_proj -- and the
indexer's four settings (head weights all ones, head scale 1, softmax scale
index_head_dim^-0.5, candidate window kv_len / compress_ratio).  Its
fresh-review section: one set of rotary angles serves the query side and
the pooled indexer keys.  The indexer takes the rotated indexer query and
the raw indexer keys; pooling comes before the pooled key's rotation.

Readings where the pages are silent (each also in the design notes):
  * weights are Linear [out][in]; one input matrix stacks the rows of the q,
    gate, k, v, indexer-q and indexer-k projections in that order;
  * the gate is a projection of its own, sigmoid-applied elementwise;
  * the q/k norm is RMSNorm over each head's D values, x / sqrt(mean(x^2) +
    eps) * (1 + w), with one [D] weight shared by all heads;
  * RoPE is the rotate-half form on the first rotary_dim values of each
    head (qsa_oracle_rope), at the token's position; the indexer query gets
    its own rotary dims, each pooled key the same angles at its block's
    first position (inside qsa_oracle_sequence);
  * the indexer has no norm and no head-weight projection (weights all ones).

Precision: the projections are fp64 matrix products of the bf16 inputs,
rounded to fp32; the norm is fp64, rounded to fp32; RoPE is the fp32
rotation of qsa_oracle_rope.  Every tensor the path stores in bf16 (q, k, v,
gate, indexer q and k, the attention output before o_proj) is rounded to
bf16 here at the same point, so that both sides see values of the same
precision.  The attention itself is the oracle's (fp64, rounded to fp32).
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def bf16_round(x) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 (ties to even), as fp32."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(np.shape(x))


def widen(x) -> np.ndarray:
    """bf16 bits (uint16) or floats -> fp32 values."""
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return np.asarray(a, np.float32)


def project(x, W) -> np.ndarray:
    """x [n][in] times W [out][in] transposed: fp64 products, rounded to fp32."""
    return (widen(x).astype(np.float64) @ widen(W).astype(np.float64).T).astype(np.float32)


def rms_norm(x, w, eps: float) -> np.ndarray:
    """RMSNorm over the last axis with the (1 + w) weight: fp64, rounded to fp32."""
    x64 = np.asarray(x, np.float64)
    ms = np.mean(x64 * x64, axis=-1, keepdims=True)
    y = x64 / np.sqrt(ms + float(eps)) * (1.0 + widen(w).astype(np.float64))
    return y.astype(np.float32)


def split_rows(bd: dict) -> dict:
    """Row ranges of the stacked input projection."""
    Hq, Hkv, D = bd["n_q_heads"], bd["n_kv_heads"], bd["head_dim"]
    HI, dI = bd["n_idx_heads"], bd["idx_dim"]
    sizes = [("q", Hq * D), ("gate", Hq * D), ("k", Hkv * D), ("v", Hkv * D),
             ("qI", HI * dI if bd["block_size"] > 0 else 0),
             ("kI", dI if bd["block_size"] > 0 else 0)]
    out, o = {}, 0
    for name, n in sizes:
        out[name] = (o, o + n)
        o += n
    out["total"] = o
    return out


def front(orc, bd: dict, x, W_in, qn_w, kn_w, pos, parts=("q", "gate", "k", "v", "qI", "kI")):
    """Projected, normed and rotated bf16-valued tensors of tokens at `pos`
    (x [n][d_model]).  Returns fp32 arrays of bf16 values: q/gate
    [n][Hq][D], k/v [n][Hkv][D], qI [n][H_I][d_I], kI [n][d_I]."""
    rows = split_rows(bd)
    Hq, Hkv, D = bd["n_q_heads"], bd["n_kv_heads"], bd["head_dim"]
    HI, dI = bd["n_idx_heads"], bd["idx_dim"]
    n = widen(x).shape[0]
    pos = np.asarray(pos, np.int64)
    W = widen(W_in)
    res = {}
    for name in parts:
        a, b = rows[name]
        if b == a:
            res[name] = None
            continue
        P = project(x, W[a:b])
        if name in ("q", "k"):
            H = Hq if name == "q" else Hkv
            t = rms_norm(P.reshape(n, H, D), qn_w if name == "q" else kn_w, bd["norm_eps"])
            t = orc.rope(t, bd["rotary_dim"], bd["rope_theta"], pos[:, None])
        elif name == "qI":
            t = orc.rope(P.reshape(n, HI, dI), bd["idx_rope_dim"], bd["idx_rope_theta"],
                         pos[:, None])
        elif name in ("gate", "v"):
            t = P.reshape(n, Hq if name == "gate" else Hkv, D)
        else:  # kI: raw, pooled and rotated inside the sequence oracle
            t = P.reshape(n, dI)
        res[name] = bf16_round(t)
    return res


def core_dims(bd: dict) -> dict:
    keys = ("n_q_heads", "n_kv_heads", "head_dim", "n_idx_heads", "idx_dim", "block_size",
            "budget", "attn_scale", "idx_scale", "idx_rope_dim", "idx_rope_theta")
    return {k: bd.get(k, 0) for k in keys}


def block(orc, bd: dict, x, W_in, qn_w, kn_w, W_o, q_pos, want_scores: bool = False,
          nb_cap: Optional[int] = None, kv8: Optional[tuple] = None) -> dict:
    """The QSA block for the queries at positions q_pos of ONE sequence whose
    tokens 0..n-1 have hidden states x [n][d_model] (the caches hold all of
    them).  Returns y [nq][d_model] (fp32), the selections, the
    intermediate bf16-valued tensors of the queries ("front") and the k, v
    and indexer-key rows of every token ("front_kv").  kv8 = (rotate,
    k_scale, v_scale): the K/V cache holds 8-bit codes of the block's k and
    v (the oracle's own encoding, qsa_oracle_kv8_encode)."""
    x = widen(x)
    n = x.shape[0]
    q_pos = np.asarray(q_pos, np.int64)
    kv = front(orc, bd, x, W_in, qn_w, kn_w, np.arange(n), parts=("k", "v", "kI"))
    qs = front(orc, bd, x[q_pos], W_in, qn_w, kn_w, q_pos, parts=("q", "gate", "qI"))
    nq = q_pos.size
    HI = bd["n_idx_heads"]
    w = np.ones((nq, max(HI, 1)), np.float32) if bd["block_size"] > 0 else None
    if kv8 is None:
        ref = orc.sequence(core_dims(bd), kv["k"], kv["v"], kv["kI"], q_pos, qs["q"], qs["qI"], w,
                           qs["gate"], want_scores=want_scores, nb_cap=nb_cap)
    else:
        rotate, ks, vs = kv8
        inv = lambda sc: float(np.float32(1.0) / np.float32(sc))  # noqa: E731
        Kc = orc.kv8_encode(kv["k"], rotate, inv(ks))
        Vc = orc.kv8_encode(kv["v"], rotate, inv(vs))
        ref = orc.sequence_kv8(core_dims(bd), Kc, Vc, rotate, ks, vs, kv["kI"], q_pos, qs["q"],
                               qs["qI"], w, qs["gate"], want_scores=want_scores, nb_cap=nb_cap)
    attn = bf16_round(ref["out"]).reshape(nq, -1)
    ref["attn"] = attn
    ref["y"] = project(attn, W_o)
    ref["front"] = qs
    ref["front_kv"] = kv
    return ref
