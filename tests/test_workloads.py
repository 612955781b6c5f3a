"""The seeded workload generator (host only): call schedules and shapes,
including the speculative-verification and dense draft-layer workloads."""
import numpy as np

from block_sparse_attention_keys_amd import workloads


def test_decode_calls_one_token_per_step():
    case = workloads.make_case("ragged_paged_decode_128k_bf16", n_seqs=3,
                               ctx_range=(100, 300), steps=4)
    for i, call in enumerate(case.calls):
        for b, (s, e) in enumerate(call):
            assert (s, e) == (case.ctx[b] + i, case.ctx[b] + i + 1)
    for b in range(3):
        assert case.k[b].shape[0] == case.ctx[b] + 4
        assert case.q[b].shape[0] == 4
        assert np.array_equal(case.q_pos[b], np.arange(case.ctx[b], case.ctx[b] + 4))


def test_spec_verify_calls_append_several_tokens():
    """Each call appends q_per_step consecutive tokens per sequence; every new
    token is a query at its own position."""
    case = workloads.make_case("spec_verify_ragged_bf16", n_seqs=3, ctx_range=(100, 300),
                               steps=3)
    m = case.spec.q_per_step
    assert m == 4
    for i, call in enumerate(case.calls):
        for b, (s, e) in enumerate(call):
            assert (s, e) == (case.ctx[b] + i * m, case.ctx[b] + (i + 1) * m)
    for b in range(3):
        assert case.k[b].shape[0] == case.ctx[b] + 3 * m
        assert case.q[b].shape[0] == 3 * m
        assert np.array_equal(case.q_pos[b], np.arange(case.ctx[b], case.ctx[b] + 3 * m))
    # paged: every token's page is mapped, physical pages are distinct
    pt = case.page_table
    used = pt[pt >= 0]
    assert used.size == np.unique(used).size == case.n_pages
    for b in range(3):
        assert np.all(pt[b, :(case.k[b].shape[0] + 63) // 64] >= 0)


def test_dense_draft_layer_workload():
    case = workloads.make_case("mtp_dense_ragged_bf16", n_seqs=2, ctx_range=(100, 300))
    assert case.spec.block_size == 0 and case.spec.k_blocks == 0
    assert all(p.size == 0 for p in case.planted)


def test_draws_do_not_depend_on_batch_layout():
    """A sequence's tensors come from its own seeded streams."""
    a = workloads.make_case("decode_32k_bf16", ctx=500, steps=2)
    b = workloads.make_case("decode_32k_bf16", ctx=500, steps=2)
    for x, y in zip((a.k, a.v, a.kI, a.q, a.qI, a.w, a.gate), (b.k, b.v, b.kI, b.q, b.qI, b.w, b.gate)):
        assert np.array_equal(x[0], y[0])
