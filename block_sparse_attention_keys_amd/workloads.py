"""Seeded synthetic workloads for Qwen Sparse Attention (QSA).

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no pooling, scoring, selection or attention).  Both the
HIP path and the CPU oracle are fed from it.

Recipe (every workload, one seed):

* ``numpy.random.SeedSequence(seed)`` spawns one child per sequence, and each
  child spawns one stream per tensor (k, v, k_I, q, q_I, w, gate, planting), so
  the values do not depend on how many threads draw them.
* q, k, v ~ N(0,1)/sqrt(D); indexer q_I, k_I ~ N(0,1)/sqrt(d_I);
  indexer head weights w ~ U(0,1) (always fp32); gate logits ~ N(0,1)
  (the kernels apply the sigmoid).
* Planted blocks: every indexer key of a planted block gets +1.5 * u_b added,
  u_b a random unit vector of R^{d_I} drawn per block.
* bf16 workloads are drawn in fp32 and rounded once to bf16 (round to nearest
  even, through torch on the CPU); both sides see the same rounded bits
  (stored here as uint16).
* Decode workloads: a sequence holds ``ctx`` cached tokens (positions
  0..ctx-1) and each step appends ``q_per_step`` new tokens (one, or several
  for speculative verification), which are also the queries.
  Prefill workloads: every token is a query; tokens arrive in chunks.

The five workloads follow the QSA description on the Qwen4-Exp pages (MTPLX
"Native Backend Components" page, section "Qwen Sparse Attention (QSA)"; the
dev.to Qwen4-Exp article, section "Qwen Sparse Attention"): block size equals
the compression ratio, the budget is in tokens, k = budget / block size.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Dict, List, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and structure of one workload."""

    name: str
    kind: str                 # "prefill" or "decode"
    dtype: str                # F32 or BF16
    n_seqs: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_idx_heads: int
    idx_dim: int
    block_size: int           # r (the pages' compression ratio)
    budget: int               # tokens; k = budget // r
    # prefill: total tokens and chunk length
    prefill_len: int = 0
    chunk: int = 0
    # decode: cached context per sequence (fixed) or a U[lo, hi] draw
    ctx: int = 0
    ctx_lo: int = 0
    ctx_hi: int = 0
    steps: int = 1
    q_per_step: int = 1       # decode: new tokens per sequence per call (speculative verify)
    # paged KV (0 = contiguous)
    page_size: int = 0
    # planting
    planted: int = 0                  # number of planted blocks per sequence
    planted_spread: bool = False      # True: block ids 8 + 16 i; else random
    planted_density: float = 0.0      # fraction of candidate blocks (overrides planted)
    # K/V cache storage: 8-bit E4M3 codes with per-tensor scales, optionally
    # in the Hadamard-rotated basis (False: the compute dtype)
    kv_fp8: bool = False
    kv_rotate: bool = False

    @property
    def k_blocks(self) -> int:
        return self.budget // self.block_size if self.block_size > 0 else 0


def kv_scales(head_dim: int, rotate: bool) -> tuple:
    """Per-tensor scales (k_scale, v_scale) of an 8-bit K/V cache for the
    draws below (K, V ~ N(0, 1/D); the rotated values H x ~ N(0, 1)): eight
    standard deviations of the stored values map to E4M3's largest finite
    value 448, so no draw saturates in practice."""
    sd = 1.0 if rotate else head_dim ** -0.5
    s = float(np.float32(8.0 * sd / 448.0))
    return s, s


SPECS: Dict[str, Spec] = {
    "tiny_prefill_f32": Spec(
        name="tiny_prefill_f32", kind="prefill", dtype=F32, n_seqs=1,
        n_q_heads=4, n_kv_heads=1, head_dim=64, n_idx_heads=2, idx_dim=32,
        block_size=16, budget=128, prefill_len=512, chunk=512, planted=4),
    "decode_32k_bf16": Spec(
        name="decode_32k_bf16", kind="decode", dtype=BF16, n_seqs=1,
        n_q_heads=16, n_kv_heads=2, head_dim=128, n_idx_heads=4, idx_dim=64,
        block_size=64, budget=2048, ctx=32768, steps=1, planted=32,
        planted_spread=True),
    "chunked_prefill_32k_bf16": Spec(
        name="chunked_prefill_32k_bf16", kind="prefill", dtype=BF16, n_seqs=1,
        n_q_heads=16, n_kv_heads=2, head_dim=128, n_idx_heads=4, idx_dim=64,
        block_size=64, budget=2048, prefill_len=32768, chunk=4096,
        planted_density=0.01),
    "ragged_paged_decode_128k_bf16": Spec(
        name="ragged_paged_decode_128k_bf16", kind="decode", dtype=BF16, n_seqs=32,
        n_q_heads=16, n_kv_heads=2, head_dim=128, n_idx_heads=4, idx_dim=64,
        block_size=64, budget=4096, ctx_lo=8192, ctx_hi=131072, steps=1,
        page_size=64),
    "long_decode_256k_bf16": Spec(
        name="long_decode_256k_bf16", kind="decode", dtype=BF16, n_seqs=4,
        n_q_heads=32, n_kv_heads=4, head_dim=128, n_idx_heads=8, idx_dim=64,
        block_size=128, budget=4096, ctx=262144, steps=128, planted=64),
    # Beyond the five configurations: speculative decoding.  A draft head
    # proposes tokens that the QSA layers then verify in one call per
    # sequence (several new tokens, each its own query with its own causal
    # selection), and the draft head's own layer attends densely (block size
    # 0).  Same batch, contexts and paging as the ragged decode.
    "spec_verify_ragged_bf16": Spec(
        name="spec_verify_ragged_bf16", kind="decode", dtype=BF16, n_seqs=32,
        n_q_heads=16, n_kv_heads=2, head_dim=128, n_idx_heads=4, idx_dim=64,
        block_size=64, budget=4096, ctx_lo=8192, ctx_hi=131072, steps=1,
        q_per_step=4, page_size=64),
    # The ragged decode with the K/V cache stored as 8-bit E4M3 codes in the
    # Hadamard-rotated basis (the quantized-KV storage contract).
    "ragged_paged_decode_128k_fp8kv": Spec(
        name="ragged_paged_decode_128k_fp8kv", kind="decode", dtype=BF16, n_seqs=32,
        n_q_heads=16, n_kv_heads=2, head_dim=128, n_idx_heads=4, idx_dim=64,
        block_size=64, budget=4096, ctx_lo=8192, ctx_hi=131072, steps=1,
        page_size=64, kv_fp8=True, kv_rotate=True),
    # The 32K chunked prefill over the 8-bit rotated K/V cache.
    "chunked_prefill_32k_fp8kv": Spec(
        name="chunked_prefill_32k_fp8kv", kind="prefill", dtype=BF16, n_seqs=1,
        n_q_heads=16, n_kv_heads=2, head_dim=128, n_idx_heads=4, idx_dim=64,
        block_size=64, budget=2048, prefill_len=32768, chunk=4096,
        planted_density=0.01, kv_fp8=True, kv_rotate=True),
    "mtp_dense_ragged_bf16": Spec(
        name="mtp_dense_ragged_bf16", kind="decode", dtype=BF16, n_seqs=32,
        n_q_heads=16, n_kv_heads=2, head_dim=128, n_idx_heads=4, idx_dim=64,
        block_size=0, budget=0, ctx_lo=8192, ctx_hi=131072, steps=1,
        page_size=64),
}

ORDER = ["tiny_prefill_f32", "decode_32k_bf16", "chunked_prefill_32k_bf16",
         "ragged_paged_decode_128k_bf16", "long_decode_256k_bf16"]


@dataclasses.dataclass
class Case:
    """Host arrays of one workload.

    Per sequence b (lists indexed by b):
      k[b], v[b]   [n_tok_b, Hkv, D]   float32 or uint16 (bf16 bits)
      kI[b]        [n_tok_b, d_I]       same dtype
      q[b], gate[b][n_q_b, Hq, D]; qI[b] [n_q_b, H_I, d_I]; w[b] [n_q_b, H_I] f32
      q_pos[b]     [n_q_b] int64 positions of the query tokens (ascending)
      ctx[b]       tokens cached before the first call
      planted[b]   planted block ids
    calls: list of per-call lists [(start, end)] per sequence -- the new token
      positions appended (and queried) by that call.
    page_perm: physical page of every logical page, per sequence (paged only).
    """

    spec: Spec
    k: List[np.ndarray]
    v: List[np.ndarray]
    kI: List[np.ndarray]
    q: List[np.ndarray]
    qI: List[np.ndarray]
    w: List[np.ndarray]
    gate: List[np.ndarray]
    q_pos: List[np.ndarray]
    ctx: List[int]
    planted: List[np.ndarray]
    calls: List[List[tuple]]
    page_table: Optional[np.ndarray] = None   # [B][max_pages] int32
    n_pages: int = 0

    @property
    def n_tok(self) -> List[int]:
        return [int(x.shape[0]) for x in self.k]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even, via torch) and return the raw bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(x: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits (uint16) to float32."""
    return (x.astype(np.uint32) << 16).view(np.float32)


def as_f32(x: np.ndarray) -> np.ndarray:
    return bits_to_f32(x) if x.dtype == np.uint16 else np.asarray(x, np.float32)


def _normal(rng, shape, scale, dtype):
    a = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return bf16_bits(a) if dtype == BF16 else a


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_case(name: str, seed: int = 0, *, ctx: Optional[int] = None,
              prefill_len: Optional[int] = None, chunk: Optional[int] = None,
              steps: Optional[int] = None, n_seqs: Optional[int] = None,
              ctx_range: Optional[tuple] = None, budget: Optional[int] = None) -> Case:
    """Draw workload ``name``; keyword overrides shrink it for fast tests."""
    sp = SPECS[name]
    repl = {}
    if ctx is not None:
        repl["ctx"] = ctx
    if prefill_len is not None:
        repl["prefill_len"] = prefill_len
    if chunk is not None:
        repl["chunk"] = chunk
    if steps is not None:
        repl["steps"] = steps
    if n_seqs is not None:
        repl["n_seqs"] = n_seqs
    if ctx_range is not None:
        repl["ctx_lo"], repl["ctx_hi"] = ctx_range
    if budget is not None:
        repl["budget"] = budget
    if repl:
        sp = dataclasses.replace(sp, **repl)
    return _draw(sp, seed)


def _draw(sp: Spec, seed: int) -> Case:
    root = np.random.SeedSequence(seed)
    meta_rng, *seq_seeds = [np.random.default_rng(s) for s in root.spawn(1 + sp.n_seqs)]
    B, r = sp.n_seqs, sp.block_size
    D, dI = sp.head_dim, sp.idx_dim

    if sp.kind == "prefill":
        ctx = [0] * B
        n_new = [sp.prefill_len] * B
    else:
        if sp.ctx_hi > 0:
            ctx = [int(x) for x in meta_rng.integers(sp.ctx_lo, sp.ctx_hi + 1, size=B)]
        else:
            ctx = [sp.ctx] * B
        n_new = [sp.steps * sp.q_per_step] * B
    n_tok = [c + n for c, n in zip(ctx, n_new)]

    # Per-sequence tensor streams.
    def seq_job(b):
        rngs = [np.random.default_rng(s) for s in
                np.random.SeedSequence(seq_seeds[b].integers(2**63)).spawn(8)]
        n = n_tok[b]
        nq = n_new[b]
        k = _normal(rngs[0], (n, sp.n_kv_heads, D), D ** -0.5, sp.dtype)
        v = _normal(rngs[1], (n, sp.n_kv_heads, D), D ** -0.5, sp.dtype)
        kI32 = rngs[2].standard_normal((n, dI), dtype=np.float32) * np.float32(dI ** -0.5)
        q = _normal(rngs[3], (nq, sp.n_q_heads, D), D ** -0.5, sp.dtype)
        qI = _normal(rngs[4], (nq, sp.n_idx_heads, dI), dI ** -0.5, sp.dtype)
        w = rngs[5].random((nq, sp.n_idx_heads), dtype=np.float32)
        gate = _normal(rngs[6], (nq, sp.n_q_heads, D), 1.0, sp.dtype)
        # Planted high-relevance blocks among this sequence's complete blocks.
        nblk = n // r if r > 0 else 0
        prng = rngs[7]
        if sp.planted_density > 0:
            npl = int(round(sp.planted_density * nblk))
        else:
            npl = min(sp.planted, nblk)
        if sp.planted_spread and npl > 0:
            stride = max(1, nblk // npl)
            ids = np.array([stride // 2 + stride * i for i in range(npl)], np.int64)
            ids = ids[ids < nblk]
        elif npl > 0:
            ids = np.sort(prng.choice(nblk, size=npl, replace=False)).astype(np.int64)
        else:
            ids = np.zeros(0, np.int64)
        if ids.size:
            u = prng.standard_normal((ids.size, dI)).astype(np.float32)
            u /= np.linalg.norm(u, axis=1, keepdims=True).astype(np.float32)
            for bid, ub in zip(ids, u):
                kI32[bid * r:(bid + 1) * r] += np.float32(1.5) * ub
        kI = bf16_bits(kI32) if sp.dtype == BF16 else kI32
        q_pos = np.arange(ctx[b], n, dtype=np.int64)
        return k, v, kI, q, qI, w, gate, q_pos, ids

    with _cf.ThreadPoolExecutor(max_workers=min(_threads(), B)) as ex:
        out = list(ex.map(seq_job, range(B)))

    # Call schedule.
    calls: List[List[tuple]] = []
    if sp.kind == "prefill":
        ch = sp.chunk
        for s in range(0, sp.prefill_len, ch):
            calls.append([(s, min(s + ch, sp.prefill_len))] * B)
    else:
        m = sp.q_per_step
        for i in range(sp.steps):
            calls.append([(ctx[b] + i * m, ctx[b] + (i + 1) * m) for b in range(B)])

    page_table = None
    n_pages = 0
    if sp.page_size > 0:
        ps = sp.page_size
        pages_per_seq = [(n + ps - 1) // ps for n in n_tok]
        max_pages = max(pages_per_seq)
        n_pages = int(sum(pages_per_seq))
        perm = meta_rng.permutation(n_pages).astype(np.int32)
        page_table = np.full((B, max_pages), -1, np.int32)
        o = 0
        for b in range(B):
            page_table[b, :pages_per_seq[b]] = perm[o:o + pages_per_seq[b]]
            o += pages_per_seq[b]

    return Case(spec=sp,
                k=[o[0] for o in out], v=[o[1] for o in out], kI=[o[2] for o in out],
                q=[o[3] for o in out], qI=[o[4] for o in out], w=[o[5] for o in out],
                gate=[o[6] for o in out], q_pos=[o[7] for o in out], ctx=ctx,
                planted=[o[8] for o in out], calls=calls,
                page_table=page_table, n_pages=n_pages)


# --------------------------------------------------------------------------
# The QSA attention block around the path: hidden states and weights.
# Hidden states x ~ N(0,1) (the block's input is normalised); Linear weights
# ~ N(0, 1/fan_in) so that projections have unit variance; norm weights
# ~ 0.1 N(0,1) (applied as 1 + w).  All bf16.

@dataclasses.dataclass
class BlockCase:
    """A QSA block workload.  spec: the core dims and the batch shape;
    x[b] [n_tok_b][d_model] bf16 bits; weights as bf16 bits: w_in [n_in][d_model]
    (rows q, gate, k, v, indexer q, indexer k), q_norm / k_norm [D],
    w_o [d_model][Hq*D].  calls: per call, one (start, end) span per sequence
    (prefill chunks of the context, then one-token decode steps)."""

    spec: Spec
    d_model: int
    rotary_dim: int
    rope_theta: float
    idx_rope_dim: int
    idx_rope_theta: float
    norm_eps: float
    x: List[np.ndarray]
    w_in: np.ndarray
    q_norm: np.ndarray
    k_norm: np.ndarray
    w_o: np.ndarray
    ctx: List[int]
    calls: List[List[tuple]]

    @property
    def n_tok(self) -> List[int]:
        return [int(a.shape[0]) for a in self.x]

    def dims(self) -> dict:
        sp = self.spec
        return dict(n_q_heads=sp.n_q_heads, n_kv_heads=sp.n_kv_heads, head_dim=sp.head_dim,
                    n_idx_heads=sp.n_idx_heads, idx_dim=sp.idx_dim, block_size=sp.block_size,
                    budget=sp.budget, attn_scale=0.0, idx_scale=0.0,
                    idx_rope_dim=self.idx_rope_dim, idx_rope_theta=self.idx_rope_theta,
                    rotary_dim=self.rotary_dim, rope_theta=self.rope_theta,
                    norm_eps=self.norm_eps)


def block_n_in(sp: Spec) -> int:
    n = 2 * sp.n_q_heads * sp.head_dim + 2 * sp.n_kv_heads * sp.head_dim
    if sp.block_size > 0:
        n += sp.n_idx_heads * sp.idx_dim + sp.idx_dim
    return n


def make_block_case(name: str, seed: int = 0, *, d_model: int = 2560, rotary_dim: int = 64,
                    rope_theta: float = 1e7, idx_rope_dim: Optional[int] = None,
                    norm_eps: float = 1e-6, chunk: int = 2048, decode_steps: int = 2,
                    n_seqs: Optional[int] = None, ctx_range: Optional[tuple] = None,
                    ctx: Optional[int] = None, budget: Optional[int] = None) -> BlockCase:
    """The block over workload ``name``'s shape (heads, block size, budget,
    contexts): each sequence's context arrives in prefill chunks of `chunk`
    tokens, then `decode_steps` single-token steps follow."""
    sp = SPECS[name]
    repl = {}
    if n_seqs is not None:
        repl["n_seqs"] = n_seqs
    if ctx_range is not None:
        repl["ctx_lo"], repl["ctx_hi"] = ctx_range
    if ctx is not None:
        repl["ctx"], repl["ctx_lo"], repl["ctx_hi"] = ctx, 0, 0
    if budget is not None:
        repl["budget"] = budget
    if repl:
        sp = dataclasses.replace(sp, **repl)
    root = np.random.SeedSequence(seed)
    meta_rng, w_rng, *seq_seeds = [np.random.default_rng(s) for s in root.spawn(2 + sp.n_seqs)]
    B = sp.n_seqs
    if sp.ctx_hi > 0:
        ctxs = [int(c) for c in meta_rng.integers(sp.ctx_lo, sp.ctx_hi + 1, size=B)]
    elif sp.kind == "prefill":
        ctxs = [sp.prefill_len] * B
    else:
        ctxs = [sp.ctx] * B
    n_tok = [c + decode_steps for c in ctxs]
    x = [bf16_bits(r.standard_normal((n, d_model), dtype=np.float32))
         for r, n in zip(seq_seeds, n_tok)]
    n_in = block_n_in(sp)
    hqd = sp.n_q_heads * sp.head_dim
    w_in = bf16_bits(w_rng.standard_normal((n_in, d_model), dtype=np.float32)
                     * np.float32(d_model ** -0.5))
    q_norm = bf16_bits(w_rng.standard_normal(sp.head_dim, dtype=np.float32) * np.float32(0.1))
    k_norm = bf16_bits(w_rng.standard_normal(sp.head_dim, dtype=np.float32) * np.float32(0.1))
    w_o = bf16_bits(w_rng.standard_normal((d_model, hqd), dtype=np.float32)
                    * np.float32(hqd ** -0.5))
    calls: List[List[tuple]] = []
    for s in range(0, max(ctxs), chunk):
        calls.append([(min(s, c), min(s + chunk, c)) for c in ctxs])
    for i in range(decode_steps):
        calls.append([(c + i, c + i + 1) for c in ctxs])
    idx_rope = (sp.idx_dim if idx_rope_dim is None else idx_rope_dim) if sp.block_size > 0 else 0
    return BlockCase(spec=sp, d_model=d_model, rotary_dim=rotary_dim, rope_theta=rope_theta,
                     idx_rope_dim=idx_rope, idx_rope_theta=rope_theta if idx_rope else 0.0,
                     norm_eps=norm_eps, x=x, w_in=w_in, q_norm=q_norm, k_norm=k_norm, w_o=w_o,
                     ctx=ctxs, calls=calls)
