"""GPU parity across head groupings.  The benchmark workloads all have 8
query heads per KV head; the attention kernels are instantiated for 1, 2, 4,
8 and 16, and the prefill kernel places its workgroups by KV head when Hkv
divides the 8 XCDs (and falls back to a plain order otherwise).  Each
grouping runs a ragged paged decode, a chunked prefill on the key-stationary
path and one on the per-token MFMA prefill kernel, against the CPU oracle."""
import dataclasses

import pytest
import torch

from block_sparse_attention_keys_amd import qsa, runner, workloads
from gpu_harness import SeqF32, check_call, run_calls, say

pytestmark = pytest.mark.gpu

# (query heads, KV heads): G = 1, 2, 4, 16, and Hkv = 3 (not a divisor of 8)
HEADS = [(16, 16), (16, 8), (16, 4), (16, 1), (12, 3)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qsa.lib()
    yield


def _case(name, hq, hkv, seed=0, **repl):
    sp = dataclasses.replace(workloads.SPECS[name], n_q_heads=hq, n_kv_heads=hkv, **repl)
    return workloads._draw(sp, seed)


@pytest.mark.parametrize("hq,hkv", HEADS)
def test_decode_head_groupings(hq, hkv):
    case = _case("ragged_paged_decode_128k_bf16", hq, hkv, n_seqs=3, ctx_lo=1500, ctx_hi=7000,
                 steps=2)
    say(f"decode Hq={hq} Hkv={hkv} ctx={case.ctx}")
    dc = runner.DeviceCase(case)
    res = run_calls(dc)
    seqf = SeqF32(case)
    for i in sorted(res):
        check_call(dc, seqf, res[i])


@pytest.mark.parametrize("hq,hkv", HEADS)
def test_mfma_prefill_head_groupings(hq, hkv):
    """600-token chunks of one sequence: the key-stationary path (a sequence
    with at least 512 new tokens), then a ragged 37-token chunk."""
    case = _case("chunked_prefill_32k_bf16", hq, hkv, prefill_len=2 * 600 + 37, chunk=600)
    say(f"prefill Hq={hq} Hkv={hkv} calls={len(case.calls)}")
    dc = runner.DeviceCase(case)
    res = run_calls(dc)
    seqf = SeqF32(case)
    for i in sorted(res):
        check_call(dc, seqf, res[i], sample=48, rng_seed=i)


@pytest.mark.parametrize("hq,hkv", HEADS)
def test_per_token_mfma_prefill_head_groupings(hq, hkv):
    """Two sequences of 300-token chunks: 600 tokens per call, at least 512
    (token, KV head) units and no sequence with 512 new tokens, so the
    per-token MFMA prefill kernel runs."""
    case = _case("chunked_prefill_32k_bf16", hq, hkv, n_seqs=2, prefill_len=2 * 300 + 37,
                 chunk=300)
    say(f"per-token prefill Hq={hq} Hkv={hkv} calls={len(case.calls)}")
    dc = runner.DeviceCase(case)
    res = run_calls(dc)
    seqf = SeqF32(case)
    for i in sorted(res):
        check_call(dc, seqf, res[i], sample=48, rng_seed=i)


@pytest.mark.parametrize("hq,hkv", [(16, 16), (16, 8), (16, 4), (16, 1), (12, 3)])
def test_decode_8bit_cache_head_groupings(hq, hkv):
    """The 8-bit (E4M3) cache across head groupings: in the Hadamard basis
    where the library supports it (4 or more query heads per KV head: the
    query is rotated across lanes), plain codes otherwise, where a rotated
    cache is refused with QSA_ERR_UNSUPPORTED."""
    case = _case("ragged_paged_decode_128k_bf16", hq, hkv, n_seqs=3, ctx_lo=1500, ctx_hi=6000,
                 steps=2)
    rotate = hq // hkv >= 4
    say(f"8-bit decode Hq={hq} Hkv={hkv} rotate={rotate} ctx={case.ctx}")
    if not rotate:
        with pytest.raises(qsa.QsaError) as err:
            runner.DeviceCase(case, kv_fp8=True, kv_rotate=True)
        assert err.value.status == qsa.QSA_ERR_UNSUPPORTED
    dc = runner.DeviceCase(case, kv_fp8=True, kv_rotate=rotate)
    res = run_calls(dc)
    seqf = SeqF32(case)
    for i in sorted(res):
        check_call(dc, seqf, res[i])
