"""8-bit K/V storage on the GPU (Porting Qwen4 to llama.cpp, section
"Quantized KV Is a Representation Contract"): the caches hold OCP E4M3 codes
with per-tensor scales, optionally in the Sylvester-Hadamard-rotated basis.
The codes the library writes (qsa_store_kv for the context, qsa_forward for
new rows) must equal the oracle's encoding bit for bit, and the outputs and
selections must equal the oracle's QSA over those codes."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_keys_amd import qsa, runner, workloads
from gpu_harness import SeqF32, check_call, run_calls, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qsa.lib()
    yield


def _run(case, rotate, sample=None, keep=None, **kw):
    say(f"case {case.spec.name} seqs={case.spec.n_seqs} ctx={case.ctx[:4]} "
        f"calls={len(case.calls)} rotate={rotate}")
    dc = runner.DeviceCase(case, kv_fp8=True, kv_rotate=rotate, **kw)
    res = run_calls(dc, keep=keep)
    seqf = SeqF32(case)
    stats = [check_call(dc, seqf, res[i], sample=sample, rng_seed=i) for i in sorted(res)]
    say("  stats", stats[-1])
    return dc, seqf


def _codes_equal(dc, seqf, seqs=None):
    """Every cached row (context and appended) equals the oracle's codes."""
    case = dc.case
    for b in (range(dc.B) if seqs is None else seqs):
        n = case.n_tok[b]
        Kc, Vc = seqf.codes(b, dc)
        gk = dc.cached_rows("k", b, n).cpu().numpy()
        gv = dc.cached_rows("v", b, n).cpu().numpy()
        for name, got, ref in (("K", gk, Kc), ("V", gv, Vc)):
            bad = np.argwhere(got != ref)
            assert bad.size == 0, (f"seq {b} {name} codes differ at {len(bad)} places, first "
                                   f"{bad[:3].tolist()}: {got[tuple(bad[0])]} vs {ref[tuple(bad[0])]}")


@pytest.mark.parametrize("rotate", [False, True])
def test_ragged_paged_decode_codes_and_outputs(rotate):
    """Ragged paged decode, several steps: cache codes bit-exact (context rows
    stored by qsa_store_kv, new rows by qsa_forward), outputs and
    selections against the oracle on every query."""
    case = workloads.make_case("ragged_paged_decode_128k_bf16", n_seqs=6,
                               ctx_range=(1500, 9000), steps=3)
    dc, seqf = _run(case, rotate)
    _codes_equal(dc, seqf)


def test_short_contexts_single_split():
    """Contexts of 0 to 300 tokens (one split per unit: the output is
    un-rotated and scaled in the attention kernel itself, not the merge)."""
    case = workloads.make_case("ragged_paged_decode_128k_bf16", n_seqs=6, ctx_range=(0, 300),
                               steps=4)
    dc, seqf = _run(case, True)
    _codes_equal(dc, seqf)


def test_decode_32k_full_rotated():
    """The 32k decode at full size with the rotated 8-bit cache."""
    _run(workloads.make_case("decode_32k_bf16"), True)


def test_spec_verify_several_tokens_per_call():
    case = workloads.make_case("spec_verify_ragged_bf16", n_seqs=4, ctx_range=(3000, 7000),
                               steps=6)
    dc, seqf = _run(case, True, keep={0, 5})
    _codes_equal(dc, seqf)


def test_dense_layer_rotated():
    """Block size 0 (every token attended) over the rotated 8-bit cache."""
    case = workloads.make_case("mtp_dense_ragged_bf16", n_seqs=4, ctx_range=(2000, 6000),
                               steps=2)
    _run(case, True)


def test_chunked_prefill_rotated():
    """Chunked prefill: each chunk stores its rows and attends them in the same
    call (chunks of 700 tokens: the key-stationary path, codes turned into
    bf16 on their way to LDS, the rotated query, the merge un-rotating)."""
    case = workloads.make_case("chunked_prefill_32k_bf16", prefill_len=2048 + 45, chunk=700)
    dc, seqf = _run(case, True)
    _codes_equal(dc, seqf)


def test_chunked_prefill_unrotated_and_short_chunks():
    """The 8-bit cache without the rotation through the key-stationary path,
    and short chunks (the split-list kernel)."""
    case = workloads.make_case("chunked_prefill_32k_bf16", prefill_len=1500 + 13, chunk=600)
    dc, seqf = _run(case, False)
    _codes_equal(dc, seqf)
    case = workloads.make_case("chunked_prefill_32k_bf16", prefill_len=700, chunk=200)
    _run(case, True)


def test_chunked_prefill_32k_full_sampled():
    """The full 32K chunked prefill over the rotated 8-bit cache, 48 sampled
    queries per 4096-token chunk."""
    _run(workloads.make_case("chunked_prefill_32k_fp8kv"), True, sample=48)


def test_saturating_scales():
    """Scales 64 times too small: many values saturate at +-448 (codes 0x7E,
    0xFE), on both sides the same way."""
    case = workloads.make_case("ragged_paged_decode_128k_bf16", n_seqs=3, ctx_range=(1000, 3000),
                               steps=2)
    s = workloads.kv_scales(case.spec.head_dim, True)[0] / 64
    dc, seqf = _run(case, True, kv_scale=(s, 2 * s))
    _codes_equal(dc, seqf)
    got = dc.cached_rows("k", 0, case.n_tok[0]).cpu().numpy()
    assert np.isin(got, [0x7E, 0xFE]).mean() > 0.05


def test_store_kv_rows_match_oracle_contiguous():
    """qsa_store_kv into a contiguous cache, then a second store that
    overwrites some rows: the cache holds the latest codes."""
    case = workloads.make_case("decode_32k_bf16", ctx=777, steps=1)
    dc = runner.DeviceCase(case, layout="contiguous", kv_fp8=True, kv_rotate=True)
    seqf = SeqF32(case)
    n = case.ctx[0]
    Kc, Vc = seqf.codes(0, dc)
    assert np.array_equal(dc.cached_rows("k", 0, n).cpu().numpy(), Kc[:n])
    assert np.array_equal(dc.cached_rows("v", 0, n).cpu().numpy(), Vc[:n])
    # Store rows 100..199 again from other values (the V rows as K and K as V).
    kk = torch.from_numpy(case.v[0][100:200]).view(torch.bfloat16).cuda()
    vv = torch.from_numpy(case.k[0][100:200]).view(torch.bfloat16).cuda()
    batch = dc.batch_for([100], [100])
    st = dc.layers[0]
    qsa.qsa_store_kv(dc.params, batch, kk, vv, st["k"], st["v"])
    torch.cuda.synchronize()
    K, V, _ = seqf.get(0)
    orc = oracle.load()
    inv = float(np.float32(1.0) / np.float32(dc.k_scale))
    got = dc.cached_rows("k", 0, n).cpu().numpy()
    assert np.array_equal(got[100:200], orc.kv8_encode(V[100:200], True, inv))
    assert np.array_equal(got[:100], Kc[:100]) and np.array_equal(got[200:n], Kc[200:n])
