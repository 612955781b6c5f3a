"""Negative controls: wrong answers that the parity comparators MUST reject.

Runs on the CPU with the oracle only.  Each control is a plausible kernel
bug (zero output, a dense walk instead of the gather, a tail off by one, a
wrong KV-head map, one swapped block); if the comparator passed any of them
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
