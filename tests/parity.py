"""Parity comparators between the HIP path and the CPU oracle.

Bars (written here, used by every GPU parity test):
  selections  bit-exact; a row may differ only where the oracle's k-th and
              (k+1)-th block scores are a near tie: |s_k - s_k+1| <=
              1e-5 * max(|s_k|, |s_k+1|), or both are below 1e-5 * the row's
              largest score (a relu boundary, a tiny positive next to +0).
  outputs     bf16: max-abs <= 2e-2 and mean-abs <= 2e-3, and per (token,
              head) ||out - ref||_2 <= 2e-2 ||ref||_2 (at the workloads' data
              scale the outputs are ~1e-3, so the absolute bounds alone
              would pass an all-zero output); fp32: max-abs <= 1e-4 and the
              same relative bound at 1e-4.
  block       (qsa_block_forward: the indexer's inputs come out of bf16
              projections whose fp32 sums run in a different order on each
              side, so an indexer value can differ by one bf16 step, about
              2^-8 of it.)  A row's selection may then differ from the
              oracle's, but every block the GPU keeps must score within
              BLOCK_SCORE_REL of the row's largest score below the oracle's
              k-th score, with the same count; at most 10 % of the rows may
              differ, and outputs are compared on the rows that agree.
"""
from __future__ import annotations

import numpy as np

BF16_MAX_ABS, BF16_MEAN_ABS, BF16_REL = 2e-2, 2e-3, 2e-2
F32_MAX_ABS, F32_REL = 1e-4, 1e-4
TIE_REL = 1e-5
BLOCK_SCORE_REL = 1e-2
BLOCK_ROWS_DIFFERING = 0.10


def output_stats(got, ref) -> dict:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    num = np.sqrt((d ** 2).sum(axis=-1))
    den = np.sqrt((ref ** 2).sum(axis=-1))
    rel = num / np.maximum(den, 1e-30)
    return {"max_abs": float(np.abs(d).max()) if d.size else 0.0,
            "mean_abs": float(np.abs(d).mean()) if d.size else 0.0,
            "max_rel": float(rel.max()) if rel.size else 0.0,
            "finite": bool(np.isfinite(got).all())}


def outputs_ok(got, ref, dtype: str):
    s = output_stats(got, ref)
    if not s["finite"]:
        return False, s
    if dtype == "bf16":
        ok = (s["max_abs"] <= BF16_MAX_ABS and s["mean_abs"] <= BF16_MEAN_ABS
              and s["max_rel"] <= BF16_REL)
    else:
        ok = s["max_abs"] <= F32_MAX_ABS and s["max_rel"] <= F32_REL
    return ok, s


def near_tie(scores_row: np.ndarray, nb: int, k: int) -> bool:
    s = np.sort(np.asarray(scores_row[:nb], np.float64))[::-1]
    if nb <= k:
        return False
    a, b = s[k - 1], s[k]
    top = max(abs(s[0]), 1e-30)
    if abs(a - b) <= TIE_REL * max(abs(a), abs(b)):
        return True
    return abs(a) <= TIE_REL * top and abs(b) <= TIE_REL * top


def selections_ok(sel_gpu, nblk_gpu, sel_ref, nblk_ref, scores_ref=None, nb=None):
    """Returns (ok, n_rows_differing, n_rows_exempted)."""
    sel_gpu = np.asarray(sel_gpu)
    sel_ref = np.asarray(sel_ref)
    if not np.array_equal(np.asarray(nblk_gpu), np.asarray(nblk_ref)):
        return False, -1, 0
    diff = np.where((sel_gpu != sel_ref).any(axis=1))[0]
    exempt = 0
    for i in diff:
        if scores_ref is None or nb is None or not near_tie(scores_ref[i], int(nb[i]),
                                                            sel_ref.shape[1]):
            return False, len(diff), exempt
        exempt += 1
    return True, len(diff), exempt


def block_selection_rows(sel_gpu, nblk_gpu, sel_ref, nblk_ref, scores_ref, nb):
    """Per row: 0 = identical, 1 = differs but valid under BLOCK_SCORE_REL,
    -1 = invalid."""
    out = np.zeros(len(sel_ref), np.int32)
    for i in range(len(sel_ref)):
        if int(nblk_gpu[i]) != int(nblk_ref[i]):
            out[i] = -1
            continue
        n = int(nblk_ref[i])
        if np.array_equal(sel_gpu[i][:n], sel_ref[i][:n]):
            continue
        s = np.asarray(scores_ref[i][:int(nb[i])], np.float64)
        kth = np.sort(s)[::-1][n - 1]
        tol = BLOCK_SCORE_REL * max(abs(s).max(), 1e-30)
        got = np.asarray(sel_gpu[i][:n])
        ok = (len(np.unique(got)) == n and (got >= 0).all() and (got < len(s)).all()
              and (s[got] >= kth - tol).all())
        out[i] = 1 if ok else -1
    return out
