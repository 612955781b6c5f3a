"""Indexer-cache lifecycle through the stateless C ABI (GPU).

The library keeps no per-sequence state: the caller's K/V cache, indexer-key
cache and pooled cache are the whole state.  Snapshot/restore, reusing a
sequence slot for another sequence and shifting a context are therefore the
caller's copies plus, where pooled blocks change, a re-pool with
``qsa_pool_keys`` (Porting, section on the indexer cache's memory contract:
the side cache follows the KV cache row for row).  These tests run those
procedures and compare the next steps with the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import parity
from block_sparse_attention_keys_amd import qsa, runner, workloads
from gpu_harness import SeqF32, check_call, dims_of, run_calls, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qsa.lib()
    yield


def _dev(a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def _step(dc, pos, q, k_new, v_new, qI, kI_new, w, gate):
    """One decode call: sequence b appends one token at pos[b]."""
    B = dc.B
    batch = dc.batch_for(list(pos), [1] * B)
    T = B
    out = torch.empty((T, dc.spec.n_q_heads, dc.spec.head_dim), dtype=dc.dt, device="cuda")
    k = dc.params.budget // dc.r
    sel = torch.empty((T, k), dtype=torch.int32, device="cuda")
    nbl = torch.empty((T,), dtype=torch.int32, device="cuda")
    ws = torch.zeros((max(qsa.qsa_workspace_size(dc.params, batch), 16),), dtype=torch.uint8,
                     device="cuda")
    st = dc.layers[0]
    qsa.qsa_forward(dc.params, batch, _dev(q), _dev(k_new), _dev(v_new), _dev(qI), _dev(kI_new),
                    _dev(w), _dev(gate), st["k"], st["v"], st["kI"], st["pooled"], out, sel, nbl,
                    ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), sel.cpu().numpy(), nbl.cpu().numpy()


def _oracle_one(dc, K, V, kI, p, q, qI, w, gate):
    orc = oracle.load()
    return orc.sequence(dims_of(dc), K, V, kI, np.array([p]), q[None], qI[None], w[None],
                        gate[None], want_scores=True)


def _check_one(dc, got_out, got_sel, got_nb, K, V, kI, p, q, qI, w, gate):
    ref = _oracle_one(dc, K, V, kI, p, q, qI, w, gate)
    ok, st = parity.outputs_ok(got_out[None], ref["out"], dc.spec.dtype)
    assert ok, st
    k = ref["sel"].shape[1]
    oks, ndiff, _ = parity.selections_ok(got_sel[None, :k], np.array([got_nb]), ref["sel"],
                                         ref["n_blocks"], ref.get("scores"),
                                         np.array([(p + 1) // dc.r]))
    assert oks, f"selection differs in {ndiff} rows"


def test_snapshot_restore_replays_bit_identically():
    """Snapshot the caches after some decode steps, decode on, restore the
    snapshot and decode the same steps again: identical outputs and
    selections (no state outside the caller's buffers)."""
    case = workloads.make_case("ragged_paged_decode_128k_bf16", n_seqs=4, ctx_range=(2000, 5000),
                               steps=12)
    dc = runner.DeviceCase(case)
    run_calls(dc, calls=list(range(6)), keep=set())
    snap = {k: v.clone() for k, v in dc.layers[0].items()}
    first = run_calls(dc, calls=list(range(6, 12)))
    for k, v in snap.items():
        dc.layers[0][k].copy_(v)
    torch.cuda.synchronize()
    again = run_calls(dc, calls=list(range(6, 12)))
    for i in range(6, 12):
        for a, b in zip(first[i][:3], again[i][:3]):
            assert np.array_equal(a, b), f"call {i} differs after restore"
    check_call(dc, SeqF32(case), again[11])


def test_slot_reuse_for_another_sequence():
    """A finished sequence's slot takes a new sequence: the caller writes the
    new context's K/V and indexer rows into the slot and re-pools it with
    qsa_pool_keys (past_len 0, only that slot has tokens); the next decode
    step is checked against the oracle for both the new and the old
    sequences."""
    a = workloads.make_case("decode_32k_bf16", ctx=2500, steps=2)
    dcase = workloads.make_case("ragged_paged_decode_128k_bf16", n_seqs=3, ctx_range=(3000, 5500),
                                steps=2)
    dc = runner.DeviceCase(dcase, layout="contiguous", extra_steps=8)
    run_calls(dc, calls=[0], keep=set())
    # The new sequence (a's context, shorter than the slot) goes into slot 1.
    slot, n = 1, a.ctx[0]
    assert n + 2 <= dc.cap
    st = dc.layers[0]
    st["k"][slot, :, :n, :] = _dev(a.k[0][:n]).permute(1, 0, 2)
    st["v"][slot, :, :n, :] = _dev(a.v[0][:n]).permute(1, 0, 2)
    B = dc.B
    counts = [0] * B
    counts[slot] = n
    batch = dc.batch_for([0] * B, counts)
    qsa.qsa_pool_keys(dc.params, batch, _dev(a.kI[0][:n]), st["kI"], st["pooled"])
    torch.cuda.synchronize()
    # Next step: slot 1 decodes a's first new token, slots 0 and 2 continue.
    pos, rows = [], {}
    for b in range(B):
        if b == slot:
            pos.append(n)
            rows[b] = (a, 0, 0, n)           # case, seq, query index, token index
        else:
            p = dcase.ctx[b] + 1
            pos.append(p)
            rows[b] = (dcase, b, 1, p)
    def cat(f):  # per slot: the query index for query tensors, the token index for rows
        return np.concatenate([getattr(c, f)[s][[j if f in ("q", "qI", "w", "gate") else t]]
                               for b, (c, s, j, t) in sorted(rows.items())], 0)
    out, sel, nbl = _step(dc, pos, cat("q"), cat("k"), cat("v"), cat("qI"), cat("kI"),
                          cat("w"), cat("gate"))
    for b, (c, s, j, t) in sorted(rows.items()):
        f32 = workloads.as_f32
        say(f"  slot {b}: position {t}")
        _check_one(dc, out[b], sel[b], nbl[b], f32(c.k[s][:t + 1]), f32(c.v[s][:t + 1]),
                   f32(c.kI[s][:t + 1]), t, c.q[s][j], c.qI[s][j], c.w[s][j], c.gate[s][j])


@pytest.mark.parametrize("shift", [100, 128])
def test_context_shift_then_repool(shift):
    """Drop a sequence's first `shift` tokens: the caller moves the remaining
    K/V and indexer rows down and re-pools the slot (block boundaries move
    unless the shift is a multiple of the block size); the next decode step
    equals the oracle on the shifted sequence."""
    case = workloads.make_case("ragged_paged_decode_128k_bf16", n_seqs=2, ctx_range=(4000, 6000),
                               steps=2)
    dc = runner.DeviceCase(case, layout="contiguous")
    run_calls(dc, calls=[0], keep=set())
    st = dc.layers[0]
    B = dc.B
    new_len = []
    for b in range(B):
        n = case.ctx[b] + 1                    # rows cached after call 0
        m = n - shift
        st["k"][b, :, :m, :] = st["k"][b, :, shift:n, :].clone()
        st["v"][b, :, :m, :] = st["v"][b, :, shift:n, :].clone()
        new_len.append(m)
    kI_rows = np.concatenate([case.kI[b][shift:case.ctx[b] + 1] for b in range(B)], 0)
    batch = dc.batch_for([0] * B, new_len)
    qsa.qsa_pool_keys(dc.params, batch, _dev(kI_rows), st["kI"], st["pooled"])
    torch.cuda.synchronize()
    # Call 1's tokens, now at positions shifted down.
    j = 1
    pos = [m for m in new_len]
    q = np.concatenate([case.q[b][j:j + 1] for b in range(B)], 0)
    qI = np.concatenate([case.qI[b][j:j + 1] for b in range(B)], 0)
    w = np.concatenate([case.w[b][j:j + 1] for b in range(B)], 0)
    gate = np.concatenate([case.gate[b][j:j + 1] for b in range(B)], 0)
    t_old = [case.ctx[b] + 1 for b in range(B)]
    k_new = np.concatenate([case.k[b][t:t + 1] for b, t in enumerate(t_old)], 0)
    v_new = np.concatenate([case.v[b][t:t + 1] for b, t in enumerate(t_old)], 0)
    kI_new = np.concatenate([case.kI[b][t:t + 1] for b, t in enumerate(t_old)], 0)
    out, sel, nbl = _step(dc, pos, q, k_new, v_new, qI, kI_new, w, gate)
    for b in range(B):
        t = t_old[b]
        f32 = workloads.as_f32
        _check_one(dc, out[b], sel[b], nbl[b], f32(case.k[b][shift:t + 1]),
                   f32(case.v[b][shift:t + 1]), f32(case.kI[b][shift:t + 1]), pos[b],
                   case.q[b][j], case.qI[b][j], case.w[b][j], case.gate[b][j])
