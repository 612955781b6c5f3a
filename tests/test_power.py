"""Negative controls: wrong answers that the parity comparators MUST reject.

Runs on the CPU with the oracle only.  Each control is a plausible kernel
bug (zero output, a dense walk instead of the gather, a tail off by one, a
wrong KV-head map, one swapped block; a near-tie row that swaps a block
outside the tie band, repeats an id, leaves the range or the order; a block
selection outside the score bands); if the comparator passed any of them
the GPU parity tests would have no power (at the workloads' data scale the
outputs are ~1e-3, inside the absolute bf16 bounds).
"""
import numpy as np
import pytest

from block_sparse_attention_keys_amd import workloads
import parity


@pytest.fixture(scope="module")
def case_and_ref(oracle_lib):
    # the decode workload's shapes, context shrunk so the oracle is instant
    case = workloads.make_case("decode_32k_bf16", ctx=6000, steps=4)
    sp = case.spec
    dims = dict(n_q_heads=sp.n_q_heads, n_kv_heads=sp.n_kv_heads, head_dim=sp.head_dim,
                n_idx_heads=sp.n_idx_heads, idx_dim=sp.idx_dim, block_size=sp.block_size,
                budget=sp.budget, attn_scale=0.0, idx_scale=0.0)
    args = (case.k[0], case.v[0], case.kI[0], case.q_pos[0], case.q[0], case.qI[0], case.w[0],
            case.gate[0])
    ref = oracle_lib.sequence(dims, *args, want_scores=True)
    return case, dims, args, ref


def _as_bf16_output(x):
    return workloads.bits_to_f32(workloads.bf16_bits(np.asarray(x, np.float32)))


def test_reference_passes_itself(case_and_ref):
    case, dims, args, ref = case_and_ref
    ok, s = parity.outputs_ok(_as_bf16_output(ref["out"]), ref["out"], "bf16")
    assert ok, s


def test_zero_output_rejected(case_and_ref):
    case, dims, args, ref = case_and_ref
    ok, s = parity.outputs_ok(np.zeros_like(ref["out"]), ref["out"], "bf16")
    assert s["max_abs"] <= parity.BF16_MAX_ABS      # the absolute bounds alone would pass it
    assert not ok


def test_dense_walk_rejected(oracle_lib, case_and_ref):
    case, dims, args, ref = case_and_ref
    dense = oracle_lib.sequence(dict(dims, budget=1 << 20), *args)
    assert not parity.outputs_ok(_as_bf16_output(dense["out"]), ref["out"], "bf16")[0]


def test_tail_off_by_one_rejected(oracle_lib, case_and_ref):
    case, dims, args, ref = case_and_ref
    K, V, kI, pos, q, qI, w, gate = args
    bad = oracle_lib.sequence(dims, K, V, kI, pos - 1, q, qI, w, gate)   # tail one token short
    assert not parity.outputs_ok(_as_bf16_output(bad["out"]), ref["out"], "bf16")[0]


def test_wrong_kv_head_map_rejected(oracle_lib, case_and_ref):
    case, dims, args, ref = case_and_ref
    K, V, kI, pos, q, qI, w, gate = args
    Hq, Hkv = dims["n_q_heads"], dims["n_kv_heads"]
    perm = (np.arange(Hq) % Hkv) * (Hq // Hkv) + np.arange(Hq) // Hkv  # h -> h % Hkv mapping
    bad = oracle_lib.sequence(dims, K, V, kI, pos, q[:, perm], qI, w, gate[:, perm])
    bad_out = np.empty_like(bad["out"])
    bad_out[:, perm] = bad["out"]
    assert not parity.outputs_ok(_as_bf16_output(bad_out), ref["out"], "bf16")[0]


def test_one_swapped_block_rejected(oracle_lib, case_and_ref):
    case, dims, args, ref = case_and_ref
    K, V, kI, pos, q, qI, w, gate = args
    i = 0
    p = int(pos[i])
    sel = ref["sel"][i].copy()
    nb = (p + 1) // dims["block_size"]
    unused = sorted(set(range(nb)) - set(sel.tolist()))
    sel[5] = unused[len(unused) // 2]
    sel.sort()
    # selection comparator rejects it
    ok, _, _ = parity.selections_ok(sel[None], ref["n_blocks"][:1], ref["sel"][:1],
                                    ref["n_blocks"][:1], ref["scores"][:1], [nb])
    assert not ok
    # and the output over the swapped token set differs beyond the relative bound
    toks = oracle_lib.token_set(sel, dims["block_size"], p)
    bad = oracle_lib.attend(q[i], workloads.as_f32(K), workloads.as_f32(V), gate[i], toks,
                            dims["head_dim"] ** -0.5)
    assert not parity.outputs_ok(_as_bf16_output(bad[None]), ref["out"][:1], "bf16")[0]


def test_near_tie_rule():
    s = np.array([5.0, 3.0, 1.0 + 1e-7, 1.0, 0.5], np.float32)
    assert parity.near_tie(s, 5, 3)
    assert not parity.near_tie(np.array([5.0, 3.0, 1.1, 1.0, 0.5]), 5, 3)
    assert parity.near_tie(np.array([5.0, 3.0, 1e-9, 0.0, 0.0]), 5, 3)


# ----------------------------------------------------------------- near-tie rows
def _tie_scores():
    """Eight blocks, k = 3: blocks 2 and 5 tie exactly at the k-th score
    (the oracle keeps 2 by the lowest-index rule); block 6 is just below."""
    s = np.array([0.9, 0.1, 0.5, 0.05, 0.8, 0.5, 0.49, 0.0], np.float32)
    return s, np.array([0, 2, 4], np.int32)


def test_near_tie_swap_inside_band_accepted():
    s, ref = _tie_scores()
    ok, nd, ex = parity.selections_ok(np.array([[0, 4, 5]]), [3], ref[None], [3], s[None], [8])
    assert ok and nd == 1 and ex == [0]


@pytest.mark.parametrize("bad", [
    [0, 4, 6],    # swaps in a block below the tie band
    [2, 4, 5],    # drops the top block for the other tied one
    [0, 5, 5],    # duplicate id
    [0, 4, 8],    # id out of range
    [4, 0, 5],    # not ascending
    [0, 4, -1],   # short count
])
def test_near_tie_invalid_rows_rejected(bad):
    s, ref = _tie_scores()
    ok, _, _ = parity.selections_ok(np.array([bad]), [3], ref[None], [3], s[None], [8])
    assert not ok


def test_differing_row_without_tie_rejected():
    s = np.array([0.9, 0.1, 0.5, 0.05, 0.8, 0.45, 0.49, 0.0], np.float32)
    ok, _, _ = parity.selections_ok(np.array([[0, 4, 6]]), [3], np.array([[0, 2, 4]]), [3],
                                    s[None], [8])
    assert not ok


def test_tie_row_output_reference_is_the_gpu_selection(oracle_lib, case_and_ref):
    """A near-tie row's output is checked against the oracle's attention over
    the GPU's own selection: that reference accepts the matching output and
    rejects the output over the oracle's (different) selection."""
    from gpu_harness import attend_over_selection
    case, dims, args, ref = case_and_ref
    K, V, kI, pos, q, qI, w, gate = args
    i, p = 0, int(pos[0])
    nb = (p + 1) // dims["block_size"]
    sel = ref["sel"][i].copy()
    unused = sorted(set(range(nb)) - set(sel.tolist()))
    sel[3] = unused[0]
    sel.sort()
    n = int(ref["n_blocks"][i])
    Kf, Vf = workloads.as_f32(K), workloads.as_f32(V)
    want = attend_over_selection(oracle_lib, dims, Kf, Vf, q[i], gate[i], sel, n, p)
    assert parity.outputs_ok(_as_bf16_output(want[None]), want[None], "bf16")[0]
    assert not parity.outputs_ok(_as_bf16_output(ref["out"][:1]), want[None], "bf16")[0]


# ----------------------------------------------------------------- block front end bars
def test_one_ulp_bar():
    x = np.array([1.0, 1.5, -3.0, 0.0, 1e-3], np.float32)[:, None]   # one row per value
    ulp = parity.bf16_ulp(x)
    assert parity.within_one_ulp(x + ulp.astype(np.float32), x).all()
    assert not parity.within_one_ulp(x + 2 * ulp.astype(np.float32), x).any()
    # a value far below its row's largest gets the row slack, not its own ulp only
    row = np.array([[4.0, 1e-3]], np.float32)
    moved = row + np.float32([[0.0, 4.0 * 2.0 ** -13]])
    assert parity.within_one_ulp(moved, row).all()
    assert not parity.within_one_ulp(row + np.float32([[0.0, 4.0 * 2.0 ** -11]]), row).all()


def test_score_bands_bound_one_ulp_query_moves(oracle_lib):
    """Moving every indexer-query element by up to one bf16 ulp moves each
    block's oracle score by no more than its band."""
    rng = np.random.default_rng(3)
    HI, dI, nb = 4, 64, 200
    qI = workloads.as_f32(workloads.bf16_bits(rng.standard_normal((HI, dI), np.float32) / 8))
    pooled = rng.standard_normal((nb, dI)).astype(np.float32) / 8
    w = rng.random(HI).astype(np.float32)
    c = float(np.float32(dI ** -0.5))
    s0 = oracle_lib.scores(qI, w, pooled, c).astype(np.float64)
    bands = parity.score_bands(qI, w, pooled, c)
    ulp = parity.bf16_ulp(qI).astype(np.float32)
    worst = 0.0
    for _ in range(50):
        moved = qI + rng.integers(-1, 2, qI.shape).astype(np.float32) * ulp
        s1 = oracle_lib.scores(moved, w, pooled, c).astype(np.float64)
        worst = max(worst, float((np.abs(s1 - s0) / bands).max()))
    assert worst <= 1.0, worst


def test_banded_selection_rejects_a_far_swap(oracle_lib):
    rng = np.random.default_rng(4)
    HI, dI, nb, k = 4, 64, 120, 16
    qI = workloads.as_f32(workloads.bf16_bits(rng.standard_normal((HI, dI), np.float32) / 8))
    pooled = rng.standard_normal((nb, dI)).astype(np.float32) / 8
    w = np.ones(HI, np.float32)
    c = float(np.float32(dI ** -0.5))
    s = oracle_lib.scores(qI, w, pooled, c)
    bands = parity.score_bands(qI, w, pooled, c)
    order = np.argsort(-s.astype(np.float64), kind="stable")
    good = np.sort(order[:k]).astype(np.int32)
    assert parity.banded_row_valid(good, k, s, bands, nb)
    bad = np.sort(np.concatenate([order[1:k], order[-1:]])).astype(np.int32)  # best out, worst in
    assert not parity.banded_row_valid(bad, k, s, bands, nb)
    dup = good.copy()
    dup[1] = dup[0]
    assert not parity.banded_row_valid(dup, k, s, bands, nb)
