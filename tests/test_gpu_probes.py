"""The gather, not a mask, measured on the GPU.

The probe build of the library (libqsa_probe.so, include/qsa_probe.h) counts
every K/V cache row its attention kernels load.  The llama.cpp PR #27739
page, LocalAI QSA-block commit ("What the context length buys") states that
the block reads n_sel rows per query and KV head instead of the whole
prefix.  So after one call the counter must equal, exactly,

    sum over the call's query tokens of  Hkv * n_sel(p),
    n_sel(p) = r * min(k, nb) + (p + 1 - r * nb),   nb = (p + 1) // r,

the size of the token set: the selected complete blocks plus the tail
(p + 1 for a dense layer).  The closed form is checked against the oracle's
token-set routine on the call's own selections, then against the counter.
Every attention kernel is covered: paged decode (bf16 and 8-bit K/V), the
MFMA prefill kernel, the fp32 split kernel, the dense layer and the block.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_keys_amd import qsa, runner, workloads
from gpu_harness import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(qsa.PROBE_PATH):
        pytest.fail(f"{qsa.PROBE_PATH} is missing: build it with "
                    "`python -m block_sparse_attention_keys_amd.build`")
    torch.cuda.init()
    with qsa.probe_library() as P:
        yield P


def n_sel(p: int, r: int, k: int) -> int:
    if r == 0:
        return p + 1
    nb = (p + 1) // r
    return r * min(k, nb) + (p + 1 - r * nb)


def expected_rows(spans, r: int, k: int, hkv: int) -> int:
    return hkv * sum(n_sel(p, r, k) for s, e in spans for p in range(s, e))


def check_sizes_with_oracle(spans, sel, nblk, r: int, k: int) -> None:
    """The closed form equals the oracle's token set of the call's own
    selections (any k distinct complete blocks give the same size)."""
    orc = oracle.load()
    t = 0
    for s, e in spans:
        for p in range(s, e):
            if r > 0:
                n = int(nblk[t])
                assert n == min(k, (p + 1) // r), (p, n)
                toks = orc.token_set(sel[t][:n], r, p)
            else:
                toks = orc.token_set(np.zeros(0, np.int32), 0, p)
            assert len(toks) == n_sel(p, r, k), (p, len(toks))
            t += 1


def _count_core(P, case, calls, **kw):
    dc = runner.DeviceCase(case, **kw)
    sp = case.spec
    r = sp.block_size
    k = sp.budget // r if r else 0
    P.qsa_probe_keys_visited(1)
    for i in range(len(case.calls)):
        inp = dc.call_inputs(i)
        outs = dc.alloc_outputs(inp)
        torch.cuda.synchronize()
        assert P.qsa_probe_keys_visited(1) >= 0
        dc.forward(inp, outs)
        torch.cuda.synchronize()
        got = P.qsa_probe_keys_visited(1)
        if i not in calls:
            continue
        spans = inp["spans"]
        want = expected_rows(spans, r, k, sp.n_kv_heads)
        say(f"  call {i}: T={inp['T']} rows loaded {got}, token sets x Hkv {want}")
        check_sizes_with_oracle(spans, outs["sel"].cpu().numpy(), outs["n_blocks"].cpu().numpy(),
                                r, k)
        assert got == want, (i, got, want)


def test_decode_loads_only_selected_rows(probe):
    case = workloads.make_case("ragged_paged_decode_128k_bf16", n_seqs=6, ctx_range=(900, 9000),
                               steps=3)
    _count_core(probe, case, calls={0, 2})


def test_decode_8bit_cache_loads_only_selected_rows(probe):
    case = workloads.make_case("ragged_paged_decode_128k_fp8kv", n_seqs=4, ctx_range=(900, 6000),
                               steps=2)
    _count_core(probe, case, calls={0, 1}, kv_fp8=True, kv_rotate=True)


def test_verify_loads_only_selected_rows(probe):
    case = workloads.make_case("spec_verify_ragged_bf16", n_seqs=3, ctx_range=(1500, 5000),
                               steps=2)
    _count_core(probe, case, calls={0, 1})


def test_mfma_prefill_loads_only_selected_rows(probe):
    case = workloads.make_case("chunked_prefill_32k_bf16", prefill_len=3000 + 17, chunk=1000)
    _count_core(probe, case, calls={0, 1, 3})


def test_fp32_split_kernel_loads_only_selected_rows(probe):
    case = workloads.make_case("tiny_prefill_f32", chunk=96)
    _count_core(probe, case, calls=set(range(len(case.calls))), layout="paged")


def test_dense_layer_loads_the_whole_prefix(probe):
    case = workloads.make_case("mtp_dense_ragged_bf16", n_seqs=3, ctx_range=(500, 3000), steps=2)
    _count_core(probe, case, calls={0, 1})


def test_block_loads_only_selected_rows(probe):
    bc = workloads.make_block_case("ragged_paged_decode_128k_bf16", d_model=256, n_seqs=3,
                                   ctx_range=(700, 4000), chunk=2048, decode_steps=2)
    dc = runner.BlockDeviceCase(bc)
    dims = bc.dims()
    r = dims["block_size"]
    k = dims["budget"] // r
    for i in range(len(bc.calls)):
        c = dc.call_inputs(i)
        torch.cuda.synchronize()
        probe.qsa_probe_keys_visited(1)
        dc.forward(c)
        torch.cuda.synchronize()
        got = probe.qsa_probe_keys_visited(1)
        want = expected_rows(c["spans"], r, k, dims["n_kv_heads"])
        say(f"  block call {i}: T={c['T']} rows loaded {got}, expected {want}")
        assert got == want, (i, got, want)


def test_pages_worked_count_measured(probe):
    """The pages' worked count, measured: kv_len 3002, ratio 4, budget 2048
    select 512 of 750 blocks, so each query and KV head loads 2050 rows
    against 3002 for the dense layer; the page prints both times a factor
    of 8 (16400 and 24016, tests/golden/qsa_worked_count.json).  The
    released geometry here has 2 KV heads, so the counter reads 2 x 2050
    and 2 x 3002."""
    import json
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                       "qsa_worked_count.json")))
    case = workloads.make_case("decode_32k_bf16", ctx=3001, steps=1)
    hkv = case.spec.n_kv_heads
    assert case.spec.budget == gold["budget"] and case.calls[0][0] == (3001, 3002)
    for r, total in ((4, gold["keys_visited_qsa"]), (0, gold["keys_visited_dense"])):
        assert total % 8 == 0
        want = total // 8 * hkv
        dc = runner.DeviceCase(case, block_size=r)
        inp = dc.call_inputs(0)
        outs = dc.alloc_outputs(inp)
        torch.cuda.synchronize()
        probe.qsa_probe_keys_visited(1)
        dc.forward(inp, outs)
        torch.cuda.synchronize()
        got = probe.qsa_probe_keys_visited(1)
        say(f"  ratio {r}: rows loaded {got} = {hkv} x {got // hkv}; the pages' count {total} = 8 x "
            f"{total // 8}")
        assert got == want


@pytest.mark.parametrize("hq,hkv", [(16, 1), (16, 4), (12, 3)])
def test_mfma_prefill_placement_loads_each_unit_once(probe, hq, hkv):
    """The prefill kernel places workgroups by KV head when Hkv divides the 8
    XCDs (a plain order otherwise): every (token, KV head) unit must run
    exactly once, which the row count shows (a unit run twice writes the same
    output, so parity alone would not)."""
    import dataclasses
    sp = dataclasses.replace(workloads.SPECS["chunked_prefill_32k_bf16"], n_q_heads=hq,
                             n_kv_heads=hkv, prefill_len=2 * 600 + 37, chunk=600)
    _count_core(probe, workloads._draw(sp, 0), calls={0, 1, 2})
