"""The QSA block front end on the GPU (qsa_block_forward) and rotary indexer
keys in the core path, against the CPU oracle (oracle/block.py and the
sequence oracle with rotated pooled keys).

Rotary indexer keys with the core entry points use seeded indexer inputs,
so pooled keys, scores and selections compare bit for bit.  Through the
block, the indexer inputs come out of bf16 projections (parity.py states the
bar for that case)."""
import numpy as np
import pytest
import torch

import oracle
import parity
from oracle import block as oblock
from block_sparse_attention_keys_amd import qsa, runner, workloads
from gpu_harness import (SeqF32, attend_over_selection, check_call, kv8_values, pooled_rows,
                         run_calls, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qsa.lib()
    yield


ROPE = (64, 1e6)


def _oracle_pooled(orc, kI, r, R, theta):
    p = orc.pool(kI, r)
    return orc.rope(p, R, theta, np.arange(p.shape[0]) * r)


def test_rotated_pooled_keys_bitexact_prefill_and_decode():
    """qsa_pool_keys on the context and the decode form's pooler on new
    blocks both store the mean rotated at the block's first position, bit
    for bit; decode outputs and selections match the oracle."""
    case = workloads.make_case("ragged_paged_decode_128k_bf16", n_seqs=5, ctx_range=(1000, 6000),
                               steps=70)
    dc = runner.DeviceCase(case, idx_rope=ROPE)
    orc = oracle.load()
    got = pooled_rows(dc)
    for b in range(case.spec.n_seqs):
        ref = _oracle_pooled(orc, case.kI[b][:case.ctx[b]], 64, *ROPE)
        assert np.array_equal(got[b, :ref.shape[0]], ref), f"context pooled keys of seq {b}"
    res = run_calls(dc, keep={0, 35, 69})
    seqf = SeqF32(case)
    for i in sorted(res):
        check_call(dc, seqf, res[i])
    got = pooled_rows(dc)
    for b in range(case.spec.n_seqs):
        ref = _oracle_pooled(orc, case.kI[b], 64, *ROPE)
        assert np.array_equal(got[b, :ref.shape[0]], ref), f"decoded pooled keys of seq {b}"


def test_rotated_pooled_keys_chunked_prefill():
    case = workloads.make_case("chunked_prefill_32k_bf16", prefill_len=3000 + 17, chunk=1000)
    dc = runner.DeviceCase(case, idx_rope=(32, 5e5))
    res = run_calls(dc, keep={0, 3})
    seqf = SeqF32(case)
    for i in sorted(res):
        check_call(dc, seqf, res[i], sample=64, rng_seed=i)
    ref = _oracle_pooled(oracle.load(), case.kI[0], 64, 32, 5e5)
    assert np.array_equal(pooled_rows(dc)[0, :ref.shape[0]], ref)


def test_rotated_pooled_keys_verify_and_fp32():
    """Rotated pooled keys through the general decode form (several new
    tokens per sequence per call) and through the fp32 kernels."""
    orc = oracle.load()
    case = workloads.make_case("spec_verify_ragged_bf16", n_seqs=3, ctx_range=(2000, 5000),
                               steps=20)
    dc = runner.DeviceCase(case, idx_rope=ROPE)
    res = run_calls(dc, keep={0, 19})
    seqf = SeqF32(case)
    for i in sorted(res):
        check_call(dc, seqf, res[i])
    got = pooled_rows(dc)
    for b in range(case.spec.n_seqs):
        ref = _oracle_pooled(orc, case.kI[b], 64, *ROPE)
        assert np.array_equal(got[b, :ref.shape[0]], ref), f"pooled keys of seq {b}"
    case = workloads.make_case("tiny_prefill_f32", chunk=96)
    dc = runner.DeviceCase(case, layout="paged", idx_rope=(16, 1e4))
    res = run_calls(dc)
    seqf = SeqF32(case)
    for i in sorted(res):
        check_call(dc, seqf, res[i])
    ref = _oracle_pooled(orc, case.kI[0], 16, 16, 1e4)
    assert np.array_equal(pooled_rows(dc)[0, :ref.shape[0]], ref)


def _run_block(bc, layout="paged", keep=None, **kw):
    dc = runner.BlockDeviceCase(bc, layout=layout, **kw)
    res = {}
    for i in range(len(bc.calls)):
        c = dc.call_inputs(i)
        say(f"  block call {i}/{len(bc.calls)}: T={c['T']}")
        dc.forward(c)
        torch.cuda.synchronize()
        if keep is None or i in keep:
            res[i] = (c["y"].float().cpu().numpy(), c["sel"].cpu().numpy(),
                      c["n_blocks"].cpu().numpy(), c["spans"])
    return dc, res


def _cache_rows(dc, name, b, n):
    """Rows [0, n) of sequence b of the block's cache `name` ("k", "v": [n][Hkv][D];
    "kI": [n][d_I]) as fp32 (8-bit K/V: the codes)."""
    st = dc.st[name]
    s = torch.arange(n, device=dc.device)
    if dc.paged:
        pg = dc.page_table[b][s // dc.page_size].long()
        off = (s % dc.page_size).long()
        rows = st[pg, :, off, :] if name in ("k", "v") else st[pg, off, :]
    else:
        rows = st[b, :, :n, :].permute(1, 0, 2) if name in ("k", "v") else st[b, :n, :]
    return rows.cpu().numpy() if rows.dtype == torch.uint8 else rows.float().cpu().numpy()


def _gpu_pooled(dc, b, nb):
    return dc.st["pooled"][b].permute(1, 0)[:nb].cpu().numpy()


def _check_block(bc, dc, result, sample=None, seed=0, kv8=None):
    """One block call against the oracle (parity.py, "block").  The caches
    hold every token of the workload by now (all calls ran), and pooled rows
    never change once written, so they are what each call read."""
    orc = oracle.load()
    y, sel, nblk, spans = result
    dims = bc.dims()
    r = dims["block_size"]
    rng = np.random.default_rng(seed)
    t0 = 0
    rows = differ = 0
    stats = None
    for b, (s, e) in enumerate(spans):
        n_q = e - s
        if n_q == 0:
            continue
        idx = np.arange(n_q)
        if sample is not None and n_q > sample:
            idx = np.sort(rng.choice(n_q, size=sample, replace=False))
        pos = s + idx
        ref = oblock.block(orc, dims, bc.x[b][:e], bc.w_in, bc.q_norm, bc.k_norm, bc.w_o, pos,
                           want_scores=r > 0, kv8=kv8)
        fkv = ref["front_kv"]
        # the cache rows this sequence's tokens put there, one ulp from the oracle's
        n_all = bc.n_tok[b]
        names = ("kI",) if kv8 else ("k", "v", "kI")
        for name in names:
            if name == "kI" and r == 0:
                continue
            got = _cache_rows(dc, name, b, e)
            okm = parity.within_one_ulp(got, fkv[name])
            assert okm.all(), (f"seq {b} cache {name}: {int((~okm).sum())} elements beyond "
                               f"one bf16 ulp, first at {np.argwhere(~okm)[0].tolist()}")
        Kx, Vx = fkv["k"], fkv["v"]
        if kv8:
            rotate, ks, vs = kv8
            inv = lambda sc: float(np.float32(1.0) / np.float32(sc))  # noqa: E731
            Kx = kv8_values(orc, orc.kv8_encode(fkv["k"], rotate, inv(ks)), rotate, ks)
            Vx = kv8_values(orc, orc.kv8_encode(fkv["v"], rotate, inv(vs)), rotate, vs)
        same = np.ones(len(idx), bool)
        yref = ref["y"].copy()
        if r > 0:
            k = ref["sel"].shape[1]
            nb_all = e // r
            pooled = _gpu_pooled(dc, b, nb_all)
            kI_gpu = _cache_rows(dc, "kI", b, nb_all * r)
            want = orc.pool(kI_gpu, r)
            if dims["idx_rope_dim"]:
                want = orc.rope(want, dims["idx_rope_dim"], dims["idx_rope_theta"],
                                np.arange(nb_all) * r)
            assert np.array_equal(pooled, want), f"seq {b}: pooled keys of the GPU's own rows"
            c = dims["idx_scale"] if dims["idx_scale"] > 0 else dims["idx_dim"] ** -0.5
            c = float(np.float32(c))
            qI = ref["front"]["qI"]
            w1 = np.ones(qI.shape[1], np.float32)
            for i in range(len(idx)):
                nb = (pos[i] + 1) // r
                n_sel = min(k, nb)
                gs = sel[t0 + idx[i]][:k]
                assert int(nblk[t0 + idx[i]]) == n_sel, f"seq {b} row {i}: n_blocks"
                if np.array_equal(gs[:n_sel], ref["sel"][i][:n_sel]) and (gs[n_sel:] == -1).all():
                    continue
                same[i] = False
                sc = orc.scores(qI[i], w1, pooled[:nb], c)
                bands = parity.score_bands(qI[i], w1, pooled[:nb], c)
                assert parity.banded_row_valid(gs, n_sel, sc, bands, nb), (
                    f"seq {b} position {pos[i]}: selection outside the score bands")
                a = attend_over_selection(orc, dims, Kx, Vx, ref["front"]["q"][i],
                                          ref["front"]["gate"][i], gs, n_sel, int(pos[i]))
                yref[i] = oblock.project(oblock.bf16_round(a).reshape(1, -1), bc.w_o)[0]
            differ += int((~same).sum())
        rows += len(idx)
        ok, stats = parity.outputs_ok(y[t0 + idx], yref, "bf16")
        assert ok, f"seq {b} block outputs {stats}"
        t0 += n_q
    say(f"  rows {rows}, selections differing inside the score bands {differ}, last stats {stats}")


def test_block_prefill_then_decode_paged():
    """Ragged contexts filled by the block's own chunked prefill (2048-token
    chunks, a ragged last chunk, sequences with no tokens in some calls),
    then decode steps; d_model 512."""
    bc = workloads.make_block_case("ragged_paged_decode_128k_bf16", d_model=512, n_seqs=4,
                                   ctx_range=(700, 5000), chunk=2048, decode_steps=3)
    dc, res = _run_block(bc)
    last = len(bc.calls) - 1
    for i in sorted(res):
        _check_block(bc, dc, res[i], sample=None if i >= last - 2 else 96, seed=i)


def test_block_prefill_on_the_tiled_gemm():
    """The block's prefill-sized projections on the library's own LDS-tiled
    MFMA kernel (hipBLASLt switched off in the probe build), chunked prefill
    and a decode step against the oracle."""
    bc = workloads.make_block_case("ragged_paged_decode_128k_bf16", d_model=512, n_seqs=2,
                                   ctx_range=(900, 4000), chunk=2048, decode_steps=1)
    with qsa.probe_library() as P:
        P.qsa_probe_library_gemm(0)
        try:
            dc, res = _run_block(bc)
        finally:
            P.qsa_probe_library_gemm(1)
    for i in sorted(res):
        _check_block(bc, dc, res[i], sample=64, seed=i)


def test_block_contiguous_equals_paged_bitwise():
    bc = workloads.make_block_case("ragged_paged_decode_128k_bf16", d_model=256, n_seqs=3,
                                   ctx_range=(300, 2500), chunk=1024, decode_steps=2)
    _, a = _run_block(bc, layout="paged")
    _, b = _run_block(bc, layout="contiguous")
    for i in a:
        for x, z in zip(a[i][:3], b[i][:3]):
            assert np.array_equal(x, z), f"call {i}"


def test_block_released_width_decode():
    """d_model 2560 (the released hidden size), one 32K-context sequence:
    the prefill in 4096-token chunks and two decode steps, outputs and
    selections of the decode steps against the oracle."""
    bc = workloads.make_block_case("decode_32k_bf16", d_model=2560, chunk=4096, decode_steps=2)
    dc, res = _run_block(bc, keep={len(bc.calls) - 2, len(bc.calls) - 1})
    for i in sorted(res):
        _check_block(bc, dc, res[i])


def test_block_dense_layer():
    """Block size 0: no indexer rows in the input projection."""
    bc = workloads.make_block_case("mtp_dense_ragged_bf16", d_model=512, n_seqs=3,
                                   ctx_range=(500, 3000), chunk=1024, decode_steps=2)
    dc, res = _run_block(bc)
    for i in sorted(res):
        _check_block(bc, dc, res[i], sample=48, seed=i)


def test_block_with_rotated_8bit_cache():
    """The block over an 8-bit K/V cache in the Hadamard basis: the block's
    bf16 k and v rows are rotated, scaled and encoded on append."""
    bc = workloads.make_block_case("ragged_paged_decode_128k_bf16", d_model=512, n_seqs=3,
                                   ctx_range=(900, 4000), chunk=2048, decode_steps=2)
    dc, res = _run_block(bc, kv_fp8=True, kv_rotate=True)
    kv8 = (True, dc.k_scale, dc.v_scale)
    for i in sorted(res):
        _check_block(bc, dc, res[i], sample=64, seed=i, kv8=kv8)
