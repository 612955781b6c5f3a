"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.  Element by element at sizes the oracle finishes in
seconds (several tiles, ragged tails); sampled queries at the workloads'
full sizes, in the launch configuration the benchmark times."""
import numpy as np
import pytest
import torch

import oracle
import parity
from block_sparse_attention_keys_amd import qsa, runner, workloads
from gpu_harness import SeqF32, check_call, pooled_rows, run_calls, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qsa.lib()
    yield


def _full(case, sample=None, keep=None, layout=None, **kw):
    say(f"case {case.spec.name} seqs={case.spec.n_seqs} ctx={case.ctx[:4]} calls={len(case.calls)}")
    dc = runner.DeviceCase(case, layout=layout, **kw)
    res = run_calls(dc, keep=keep)
    seqf = SeqF32(case)
    stats = []
    for i in sorted(res):
        say(f"  checking call {i}")
        stats.append(check_call(dc, seqf, res[i], sample=sample, rng_seed=i))
    say("  stats", stats[-1])
    return dc, res, stats


# ----------------------------------------------------------------- workloads
def test_tiny_prefill_f32():
    _full(workloads.make_case("tiny_prefill_f32"))


def test_tiny_prefill_f32_chunked_paged():
    case = workloads.make_case("tiny_prefill_f32", chunk=96)   # ragged last chunk
    _full(case, layout="paged")


def test_decode_32k_full():
    _full(workloads.make_case("decode_32k_bf16"))


def test_chunked_prefill_reduced_all_queries():
    _full(workloads.make_case("chunked_prefill_32k_bf16", prefill_len=4096 + 37, chunk=1024))


def test_chunked_prefill_full_sampled():
    _full(workloads.make_case("chunked_prefill_32k_bf16"), sample=48)


def test_ragged_paged_decode_reduced():
    _full(workloads.make_case("ragged_paged_decode_128k_bf16", n_seqs=9,
                              ctx_range=(70, 9000)))


def test_ragged_paged_decode_full():
    _full(workloads.make_case("ragged_paged_decode_128k_bf16"))


def test_long_decode_reduced_crosses_block():
    case = workloads.make_case("long_decode_256k_bf16", n_seqs=2, ctx=9000 - 3, steps=140)
    dc, _, _ = _full(case)
    # the pooled cache after incremental updates equals from-scratch pooling
    orc = oracle.load()
    got = pooled_rows(dc)
    for b in range(case.spec.n_seqs):
        ref = orc.pool(case.kI[b], case.spec.block_size)
        assert np.array_equal(got[b, :ref.shape[0]], ref)


def test_paged_decode_steps_cross_blocks():
    """70 decode steps per sequence on a paged cache (one new token per
    sequence: the launch that scores also appends and pools): every sequence
    completes a block on the way, and the pooled cache equals from-scratch
    pooling of the appended rows."""
    case = workloads.make_case("ragged_paged_decode_128k_bf16", n_seqs=5, ctx_range=(30, 400),
                               steps=70)
    dc, _, _ = _full(case, layout="paged", keep={0, 1, 33, 69})
    orc = oracle.load()
    got = pooled_rows(dc)
    for b in range(case.spec.n_seqs):
        ref = orc.pool(case.kI[b], case.spec.block_size)
        assert np.array_equal(got[b, :ref.shape[0]], ref)


def test_long_decode_full_sampled_steps():
    case = workloads.make_case("long_decode_256k_bf16")
    keep = {0, 1, 64, 126, 127}
    dc, res, stats = _full(case, keep=keep)
    orc = oracle.load()
    got = pooled_rows(dc)
    r = case.spec.block_size
    for b in range(case.spec.n_seqs):
        n = case.n_tok[b]
        ref = orc.pool(case.kI[b][(n // r - 2) * r:n // r * r], r)   # last two blocks
        assert np.array_equal(got[b, n // r - 2:n // r], ref)


def test_paged_cache_over_4gib():
    """K and V page pools of 4.3 GB each (rows past 2^24): the decode kernel
    addresses them with 64-bit pointers instead of buffer offsets."""
    case = workloads.make_case("ragged_paged_decode_128k_bf16", n_seqs=4, ctx_range=(2000, 9000))
    _full(case, layout="paged", page_offset=131072)
    torch.cuda.empty_cache()


def test_spec_verify_paged_several_tokens_per_call():
    """Speculative verification: each call appends 4 tokens per sequence on a
    paged cache (each its own query with its own selection); every sequence
    completes blocks inside a call, and the pooled cache equals from-scratch
    pooling at the end."""
    case = workloads.make_case("spec_verify_ragged_bf16", n_seqs=5, ctx_range=(3000, 9000),
                               steps=20)
    dc, _, _ = _full(case, keep={0, 1, 9, 19})
    orc = oracle.load()
    got = pooled_rows(dc)
    for b in range(case.spec.n_seqs):
        ref = orc.pool(case.kI[b], case.spec.block_size)
        assert np.array_equal(got[b, :ref.shape[0]], ref)


def test_dense_draft_layer_paged_decode():
    """The draft head's dense layer (block size 0) decoding over ragged paged
    contexts."""
    _full(workloads.make_case("mtp_dense_ragged_bf16", n_seqs=4, ctx_range=(2000, 7000),
                              steps=2))


def test_dense_long_context_several_rounds():
    """A dense layer over 140000 cached tokens: each split holds more list
    positions than one round of row resolution."""
    case = workloads.make_case("decode_32k_bf16", ctx=140000, steps=1)
    dc = runner.DeviceCase(case, block_size=0)
    res = run_calls(dc)
    check_call(dc, SeqF32(case), res[0])


def test_selection_ties_all_scores_equal():
    """Zero indexer queries: every candidate block scores 0, so the selection
    is the tie rule alone (the lowest block ids)."""
    case = workloads.make_case("decode_32k_bf16", ctx=9000, steps=2)
    for b in range(case.spec.n_seqs):
        case.qI[b][:] = 0
    _full(case)


def test_selection_ties_at_the_boundary():
    """Indexer keys with a negative first dimension except in five blocks,
    and queries that read only that dimension: five blocks share one positive
    score and all others score 0, so the k-th largest score is a tie broken
    by block id."""
    case = workloads.make_case("decode_32k_bf16", ctx=9000, steps=2)
    r = case.spec.block_size
    for b in range(case.spec.n_seqs):
        kI = workloads.as_f32(case.kI[b]).copy()
        kI[:, 0] = -1.0
        for blk in (3, 10, 50, 77, 100):
            kI[blk * r:(blk + 1) * r, 0] = 1.0
        case.kI[b] = workloads.bf16_bits(kI)
        qI = np.zeros(case.qI[b].shape, np.float32)
        qI[..., 0] = 1.0
        case.qI[b] = workloads.bf16_bits(qI)
    _full(case)


def test_prefill_selection_ties_all_scores_equal():
    """The prefill form of the all-equal case: zero indexer queries over a
    chunked prefill whose later queries have more candidate blocks than k,
    so the selection of those queries is the tie rule alone."""
    case = workloads.make_case("chunked_prefill_32k_bf16", prefill_len=4096 + 37, chunk=1024)
    for b in range(case.spec.n_seqs):
        case.qI[b][:] = 0
    _full(case)


def test_prefill_selection_ties_at_the_boundary():
    """The prefill form of the boundary tie: five blocks share one positive
    score, all others score 0, and k = 32 lies inside the zeros."""
    case = workloads.make_case("chunked_prefill_32k_bf16", prefill_len=4096 + 37, chunk=1024)
    r = case.spec.block_size
    for b in range(case.spec.n_seqs):
        kI = workloads.as_f32(case.kI[b]).copy()
        kI[:, 0] = -1.0
        for blk in (3, 10, 40, 51, 60):
            kI[blk * r:(blk + 1) * r, 0] = 1.0
        case.kI[b] = workloads.bf16_bits(kI)
        qI = np.zeros(case.qI[b].shape, np.float32)
        qI[..., 0] = 1.0
        case.qI[b] = workloads.bf16_bits(qI)
    _full(case)


@pytest.mark.parametrize("extra", [0, 40000, 140000])
def test_prefill_selection_tie_classes_every_select_path(extra):
    """Indexer keys that repeat one of three patterns block by block, so that
    a query's scores take at most three values and its k-th score is shared
    by many blocks: inside that class the selection is the tie rule alone.
    Cache capacities of 4.1K, 44K and 144K tokens make the score rows 64,
    689 and 2252 candidates wide, which puts them on each of the three
    selection kernels (a wave per query; a workgroup per query with the keys
    in registers; the keys in memory) and the plan on both of its forms."""
    case = workloads.make_case("chunked_prefill_32k_bf16", prefill_len=4096 + 37, chunk=1024)
    r = case.spec.block_size
    rng = np.random.default_rng(7)
    for b in range(case.spec.n_seqs):
        kI = workloads.as_f32(case.kI[b]).copy()
        pats = rng.integers(-2, 3, size=(3, kI.shape[1])).astype(np.float32) * 0.25
        cls = rng.integers(0, 3, size=kI.shape[0] // r)
        for blk, c in enumerate(cls):
            kI[blk * r:(blk + 1) * r] = pats[c]
        case.kI[b] = workloads.bf16_bits(kI)
    _full(case, extra_steps=extra)


def test_decode_selection_tie_classes():
    """The tie classes of the prefill test above through the decode path,
    where every attention workgroup makes the selection itself: ragged paged
    contexts with up to 140 candidate blocks, k = 64."""
    case = workloads.make_case("ragged_paged_decode_128k_bf16", n_seqs=9, ctx_range=(70, 9000),
                               steps=3)
    r = case.spec.block_size
    rng = np.random.default_rng(11)
    for b in range(case.spec.n_seqs):
        kI = workloads.as_f32(case.kI[b]).copy()
        pats = rng.integers(-2, 3, size=(3, kI.shape[1])).astype(np.float32) * 0.25
        cls = rng.integers(0, 3, size=kI.shape[0] // r)
        for blk, c in enumerate(cls):
            kI[blk * r:(blk + 1) * r] = pats[c]
        case.kI[b] = workloads.bf16_bits(kI)
    _full(case, layout="paged")


# ----------------------------------------------------------------- the pages' case
def test_pages_worked_count_released_config():
    """kv_len 3002, ratio 4, budget 2048: 512 of 750 blocks and 2050 keys
    (LocalAI QSA-block commit, section on the context length)."""
    sp = workloads.SPECS["decode_32k_bf16"]
    case = workloads.make_case("decode_32k_bf16", ctx=3001, steps=1)
    dc = runner.DeviceCase(case, block_size=4)
    res = run_calls(dc)
    out, sel, nblk, spans = res[0]
    assert nblk[0] == 512
    n_tok = 4 * int(nblk[0]) + (3002 - 4 * (3002 // 4))
    assert n_tok == 2050 and 8 * n_tok == 16400
    check_call(dc, SeqF32(case), res[0])


# ----------------------------------------------------------------- modes and edges
def test_dense_layer_ratio_zero():
    case = workloads.make_case("tiny_prefill_f32", chunk=200)
    dc = runner.DeviceCase(case, block_size=0)
    res = run_calls(dc)
    seqf = SeqF32(case)
    for i in res:
        check_call(dc, seqf, res[i])


def test_budget_above_context_equals_dense():
    case = workloads.make_case("decode_32k_bf16", ctx=1500, steps=3)
    a = runner.DeviceCase(case, budget=4096)
    b = runner.DeviceCase(case, block_size=0)
    ra, rb = run_calls(a), run_calls(b)
    for i in ra:
        ok, st = parity.outputs_ok(ra[i][0], rb[i][0], "bf16")
        assert ok, st
        assert (ra[i][2] == (np.array([s for s, _ in ra[i][3]]) + 1) // 64).all()


def test_paged_equals_contiguous_bitwise():
    case = workloads.make_case("ragged_paged_decode_128k_bf16", n_seqs=5, ctx_range=(100, 7000))
    a = run_calls(runner.DeviceCase(case, layout="paged"))
    b = run_calls(runner.DeviceCase(case, layout="contiguous"))
    for i in a:
        assert np.array_equal(a[i][0], b[i][0]) and np.array_equal(a[i][1], b[i][1])


def test_short_contexts_and_ragged_query_lengths():
    """Positions 0.., contexts shorter than a block, several new tokens per
    sequence with different counts in one call."""
    case = workloads.make_case("ragged_paged_decode_128k_bf16", n_seqs=6, ctx_range=(0, 200))
    case.ctx[:] = [0, 1, 63, 64, 65, 190]
    # re-cut the calls: per sequence a different number of new tokens
    n_new = [5, 1, 3, 70, 2, 9]
    for b in range(6):
        need = case.ctx[b] + n_new[b]
        assert case.k[b].shape[0] >= 1
        reps = -(-need // case.k[b].shape[0])
        for name in ("k", "v", "kI"):
            arr = getattr(case, name)
            arr[b] = np.concatenate([arr[b]] * reps)[:need]
        for name in ("q", "qI", "w", "gate"):
            arr = getattr(case, name)
            arr[b] = np.concatenate([arr[b]] * n_new[b])[:n_new[b]]
        case.q_pos[b] = np.arange(case.ctx[b], need)
    case.calls = [[(case.ctx[b], case.ctx[b] + n_new[b]) for b in range(6)]]
    case.page_table = None
    _full(case, layout="paged")


def test_nan_poison_gather_not_mask():
    """NaN in every K/V row outside each query's token set leaves the outputs
    bit-identical: the consumer gathers the selection, it does not mask a
    dense walk (LocalAI QSA-block commit, NaN-poison probe)."""
    case = workloads.make_case("decode_32k_bf16", ctx=9000, steps=1)
    dc = runner.DeviceCase(case, layout="contiguous", extra_steps=64)
    inp = dc.call_inputs(0)
    outs = dc.alloc_outputs(inp)
    dc.forward(inp, outs)
    torch.cuda.synchronize()
    base = outs["out"].clone()
    sel = outs["sel"][0].cpu().numpy()
    p = case.ctx[0]
    r = dc.r
    keep = np.zeros(dc.cap, bool)
    for j in sel[sel >= 0]:
        keep[j * r:(j + 1) * r] = True
    keep[(p + 1) // r * r:p + 1] = True
    poison = torch.from_numpy(~keep).to("cuda")
    st = dc.layers[0]
    st["k"][:, :, poison, :] = float("nan")
    st["v"][:, :, poison, :] = float("nan")
    out2 = torch.empty_like(base)
    qsa.qsa_attend(dc.params, inp["batch"], inp["q"], st["k"], st["v"], outs["sel"],
                   outs["n_blocks"], inp["gate"], out2, outs["ws"])
    torch.cuda.synchronize()
    assert torch.isfinite(out2.float()).all()
    assert torch.equal(out2, base)


def test_score_values_bitexact_and_side_cache_rows():
    """The pre-top-k scores equal the oracle's bit for bit (the value gate:
    a selection cannot see a wrong scale), and after a split prefill + decode
    the indexer side cache holds every row at its own position (not row 0)."""
    case = workloads.make_case("chunked_prefill_32k_bf16", prefill_len=1000, chunk=300)
    dc = runner.DeviceCase(case, layout="paged")
    run_calls(dc)
    orc = oracle.load()
    kI = workloads.as_f32(case.kI[0])
    # side cache row for row
    st = dc.layers[0]
    pt = dc.page_table_np[0]
    s = np.arange(case.n_tok[0])
    rows = st["kI"][torch.from_numpy(pt[s // dc.page_size]).long().cuda(),
                    torch.from_numpy(s % dc.page_size).long().cuda()].float().cpu().numpy()
    assert np.array_equal(rows, kI)
    # scores through qsa_score_select with the optional score output
    T = case.n_tok[0]
    batch = dc.batch_for([0], [T])
    qI = torch.from_numpy(case.qI[0]).view(torch.bfloat16).cuda()
    w = torch.from_numpy(case.w[0]).cuda()
    nbcap = T // dc.r
    scores = torch.empty((T, nbcap), dtype=torch.float32, device="cuda")
    k = dc.params.budget // dc.r
    sel = torch.empty((T, k), dtype=torch.int32, device="cuda")
    nbl = torch.empty((T,), dtype=torch.int32, device="cuda")
    ws = torch.zeros((qsa.qsa_workspace_size(dc.params, batch),), dtype=torch.uint8, device="cuda")
    qsa.qsa_score_select(dc.params, batch, qI, w, st["pooled"], sel, nbl, scores, ws)
    torch.cuda.synchronize()
    from gpu_harness import dims_of
    ref = orc.sequence(dims_of(dc), workloads.as_f32(case.k[0]), workloads.as_f32(case.v[0]),
                       kI, np.arange(T), case.q[0], case.qI[0], case.w[0], case.gate[0],
                       want_scores=True, nb_cap=nbcap)
    got = scores.cpu().numpy()
    assert np.array_equal(np.isneginf(got), np.isneginf(ref["scores"]))
    fin = np.isfinite(ref["scores"])
    assert np.array_equal(got[fin], ref["scores"][fin])
    assert np.array_equal(sel.cpu().numpy(), ref["sel"])


def test_zero_tokens_noop():
    case = workloads.make_case("tiny_prefill_f32", chunk=512)
    dc = runner.DeviceCase(case)
    b = dc.batch_for([0], [0])
    dummy = torch.empty(16, device="cuda")
    qsa.qsa_forward(dc.params, b, dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                    dc.layers[0]["k"], dc.layers[0]["v"], dc.layers[0]["kI"],
                    dc.layers[0]["pooled"], dummy)
    torch.cuda.synchronize()


def test_repeated_attend_reuses_workspace():
    """Repeated calls on one workspace (holding the previous call's split
    partials) give bit-identical outputs: nothing carries over between calls,
    for a plan with many splits (one decode token) and a multi-token call."""
    for name, kw in (("decode_32k_bf16", {}), ("long_decode_256k_bf16", dict(ctx=20000, steps=1)),
                     ("tiny_prefill_f32", dict(chunk=512))):
        case = workloads.make_case(name, **kw)
        dc = runner.DeviceCase(case)
        inp = dc.call_inputs(0)
        outs = dc.alloc_outputs(inp)
        dc.forward(inp, outs)
        torch.cuda.synchronize()
        first = outs["out"].clone()
        st = dc.layers[0]
        for _ in range(3):
            again = torch.empty_like(first)
            qsa.qsa_attend(dc.params, inp["batch"], inp["q"], st["k"], st["v"], outs["sel"],
                           outs["n_blocks"], inp["gate"], again, outs["ws"])
            torch.cuda.synchronize()
            assert torch.equal(again, first), name


def test_ragged_prefill_across_sub_batches():
    """Several sequences' prefill chunks in one call, more new tokens than one
    sub-batch of the key-stationary path holds: a sequence split across two
    sub-batches, and a short chunk alone in the second sub-batch."""
    import dataclasses
    sp = dataclasses.replace(workloads.SPECS["chunked_prefill_32k_bf16"], n_seqs=3,
                             prefill_len=4096)
    case = workloads._draw(sp, 0)
    case.calls = [[(0, 2048), (0, 2048), (0, 2048)],
                  [(2048, 4096), (2048, 4096), (2048, 2060)],
                  [(4096, 4096), (4096, 4096), (2060, 2100)]]
    _full(case, sample=64)
    _full(case, sample=64, layout="paged")


@pytest.mark.parametrize("n_tok", [40000, 80000, 140000])
def test_prefill_key_stationary_many_candidate_blocks(n_tok):
    """Block size 32 over 40K, 80K and 140K tokens: 1251, 2501 and 4376
    candidate blocks, so the plan's scan takes 2, 4 and 8 blocks per thread.
    One call prefills all but the last 1024 tokens (tens of sub-batches), the
    next the rest."""
    import dataclasses
    sp = dataclasses.replace(workloads.SPECS["chunked_prefill_32k_bf16"], block_size=32,
                             budget=2048, prefill_len=n_tok)
    case = workloads._draw(sp, 0)
    case.calls = [[(0, n_tok - 1024)], [(n_tok - 1024, n_tok)]]
    _full(case, sample=24)


def test_prefill_key_stationary_block_128():
    """Block size 128 with the 256K decode's heads (Hq 32, Hkv 4, indexer
    8 x 64, budget 4096: k = 32) through the key-stationary prefill, whose
    128-key blocks fill the LDS; 2048-token chunks, the last ragged, with
    more candidate blocks than k in the later chunks."""
    import dataclasses
    sp = dataclasses.replace(workloads.SPECS["chunked_prefill_32k_bf16"], n_q_heads=32,
                             n_kv_heads=4, n_idx_heads=8, block_size=128, budget=4096,
                             prefill_len=6000, chunk=2048)
    case = workloads._draw(sp, 0)
    _full(case, sample=48)
    _full(case, sample=48, layout="paged")
