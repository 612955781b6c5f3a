"""The calls are graph-capturable: no allocation, no host synchronisation,
no memset or copy nodes.  Decode and prefill steps of the path (qsa_forward)
and of the block (qsa_block_forward) are captured into a HIP graph through
torch, replayed several times with eager work and synchronisations in
between, and every replay must reproduce the eager call bit for bit (the
step rewrites the same cache rows with the same values, so replays are
idempotent)."""
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


def _replays_match(run, outs, n=3):
    run()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(n):
        for v in outs.values():
            v.fill_(0)
        junk = torch.randn(4096, device="cuda").float().sum().item()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v, ref[k]), f"replay {rep}: {k} differs from the eager call"
        say(f"  replay {rep} matches ({junk:.3f})")


def test_decode_step_graph():
    case = workloads.make_case("ragged_paged_decode_128k_bf16", n_seqs=5, ctx_range=(1000, 6000),
                               steps=1)
    dc = runner.DeviceCase(case)
    inp = dc.call_inputs(0)
    outs = dc.alloc_outputs(inp)
    ws = outs.pop("ws")
    _replays_match(lambda: dc.forward(inp, dict(outs, ws=ws)), outs)


def test_prefill_chunk_graph():
    case = workloads.make_case("chunked_prefill_32k_bf16", prefill_len=2048 + 7, chunk=1024)
    dc = runner.DeviceCase(case)
    for i in range(2):
        x = dc.call_inputs(i)
        o = dc.alloc_outputs(x)
        dc.forward(x, o)
    inp = dc.call_inputs(2)
    outs = dc.alloc_outputs(inp)
    ws = outs.pop("ws")
    _replays_match(lambda: dc.forward(inp, dict(outs, ws=ws)), outs)


def test_block_decode_step_graph():
    bc = workloads.make_block_case("ragged_paged_decode_128k_bf16", d_model=512, n_seqs=3,
                                   ctx_range=(600, 2500), chunk=4096, decode_steps=1)
    dc = runner.BlockDeviceCase(bc)
    dc.forward(dc.call_inputs(0))      # the context, through the block
    c = dc.call_inputs(1)
    outs = {"y": c["y"], "sel": c["sel"], "n_blocks": c["n_blocks"]}
    _replays_match(lambda: dc.forward(c), outs)


def test_block_prefill_chunk_graph():
    """A 2048-token block prefill step: its projections go through hipBLASLt
    (the plan was made by the eager call of the same shape before capture) and
    its attention through the key-stationary plan, attention and merge."""
    bc = workloads.make_block_case("ragged_paged_decode_128k_bf16", d_model=512, n_seqs=2,
                                   ctx_range=(2500, 3500), chunk=1024, decode_steps=1)
    dc = runner.BlockDeviceCase(bc)
    first = dc.call_inputs(0)
    assert first["T"] == 2048
    dc.forward(first)
    c = dc.call_inputs(1)
    assert c["T"] == 2048
    outs = {"y": c["y"], "sel": c["sel"], "n_blocks": c["n_blocks"]}
    _replays_match(lambda: dc.forward(c), outs)
