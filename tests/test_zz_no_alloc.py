"""The allocation-free entry point (qsa_forward_noalloc) against qsa_forward
through the C ABI: the same kernels on the same inputs, with the workspace
taken from the library's device scratch instead of a caller buffer.  Both
run on their own copy of the same caches and must agree bit for bit: the
outputs, the selections and every cache row they append.  Consecutive calls
share the scratch, so they run back to back, each smaller than the last."""
import numpy as np
import pytest
import torch

from block_sparse_attention_keys_amd import qsa, runner, workloads
from gpu_harness import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qsa.lib()
    yield


def _both(dc, i):
    """Call i through qsa_forward (cache copy 0) and qsa_forward_noalloc (copy 1)."""
    inp = dc.call_inputs(i)
    a, b = dc.alloc_outputs(inp), dc.alloc_outputs(inp)
    say(f"  call {i}: T={inp['T']}, workspace {qsa.qsa_workspace_size(dc.params, inp['batch'])} B")
    dc.forward(inp, a, layer=0)
    st = dc.layers[1]
    qsa.qsa_forward_noalloc(dc.params, inp["batch"], inp["q"], inp["k_new"], inp["v_new"],
                            inp["qI"], inp["kI_new"], inp["w"], inp["gate"], st["k"], st["v"],
                            st.get("kI"), st.get("pooled"), b["out"], b["sel"], b["n_blocks"])
    torch.cuda.synchronize()
    assert torch.equal(a["out"], b["out"]), "outputs"
    if dc.r > 0:
        assert torch.equal(a["sel"], b["sel"]) and torch.equal(a["n_blocks"], b["n_blocks"])
    for name in dc.layers[0]:
        assert torch.equal(dc.layers[0][name], dc.layers[1][name]), f"cache {name}"
    return inp["T"]


def test_noalloc_matches_forward_on_consecutive_shrinking_calls():
    big = workloads.make_case("ragged_paged_decode_128k_bf16", n_seqs=12,
                              ctx_range=(3000, 60000), steps=2)
    small = workloads.make_case("ragged_paged_decode_128k_bf16", n_seqs=3,
                                ctx_range=(500, 4000), steps=1)
    prefill = workloads.make_case("chunked_prefill_32k_bf16", prefill_len=2048 + 37, chunk=256)
    dc_big = runner.DeviceCase(big, n_layers=2)
    dc_small = runner.DeviceCase(small, n_layers=2)
    dc_pre = runner.DeviceCase(prefill, n_layers=2)
    sizes = []
    for dc, i in ((dc_pre, 0), (dc_pre, 1), (dc_big, 0), (dc_big, 1), (dc_small, 0),
                  (dc_pre, 2)):
        sizes.append(qsa.qsa_workspace_size(dc.params, dc.call_inputs(i)["batch"]))
        _both(dc, i)
    # the decode calls shrink: the 3-sequence call follows the 12-sequence one
    assert sizes[4] < sizes[3]


def test_noalloc_dense_layer_and_fp32():
    case = workloads.make_case("mtp_dense_ragged_bf16", n_seqs=4, ctx_range=(2000, 7000), steps=1)
    _both(runner.DeviceCase(case, n_layers=2), 0)
    case = workloads.make_case("tiny_prefill_f32", chunk=200)
    dc = runner.DeviceCase(case, n_layers=2)
    for i in range(len(case.calls)):
        _both(dc, i)


def test_noalloc_rejects_a_call_beyond_its_scratch():
    case = workloads.make_case("chunked_prefill_32k_bf16", prefill_len=2048, chunk=2048)
    dc = runner.DeviceCase(case)
    inp = dc.call_inputs(0)
    b = dc.batch_for([0], [8192])
    b.c.max_kv_len = 131072
    b.c.kv_capacity = 131072
    assert qsa.qsa_workspace_size(dc.params, b) > qsa.QSA_NOALLOC_SCRATCH_BYTES
    out = dc.alloc_outputs(inp)
    st = dc.layers[0]
    with pytest.raises(qsa.QsaError) as e:
        qsa.qsa_forward_noalloc(dc.params, b, inp["q"], inp["k_new"], inp["v_new"], inp["qI"],
                                inp["kI_new"], inp["w"], inp["gate"], st["k"], st["v"], st["kI"],
                                st["pooled"], out["out"], out["sel"], out["n_blocks"])
    assert e.value.status == qsa.QSA_ERR_WORKSPACE
