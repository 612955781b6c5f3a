"""Host AddressSanitizer over the CPU oracle and the C-ABI layer.

Each runs in a child process with the sanitizer runtime preloaded (the
Python interpreter itself is not instrumented): the oracle's routines on
small inputs (pooling, scores, top-k, token sets, attention, the whole
sequence, 8-bit storage), and every validation path of the C ABI that runs
without a GPU (bad parameters, bad batches, null and misaligned pointers,
short workspaces, the allocation-free entry point's size check).  A
sanitizer report fails the child and the test.  No GPU is touched."""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ORACLE_CHILD = textwrap.dedent("""
    import sys, numpy as np
    sys.path.insert(0, ROOT); sys.path.insert(0, ROOT + "/tests")
    import oracle
    from block_sparse_attention_keys_amd import workloads
    orc = oracle.load(LIB)
    rng = np.random.default_rng(0)
    kI = rng.standard_normal((333, 32)).astype(np.float32)
    P = orc.pool(kI, 16)
    s = orc.scores(rng.standard_normal((2, 32)).astype(np.float32), np.ones(2, np.float32), P, 0.2)
    sel = orc.topk(s, 8)
    toks = orc.token_set(sel, 16, 332)
    K = rng.standard_normal((333, 1, 64)).astype(np.float32)
    V = rng.standard_normal((333, 1, 64)).astype(np.float32)
    q = rng.standard_normal((4, 64)).astype(np.float32)
    out = orc.attend(q, K, V, q, toks, 0.125)
    case = workloads.make_case("tiny_prefill_f32")
    sp = case.spec
    dims = dict(n_q_heads=sp.n_q_heads, n_kv_heads=sp.n_kv_heads, head_dim=sp.head_dim,
                n_idx_heads=sp.n_idx_heads, idx_dim=sp.idx_dim, block_size=sp.block_size,
                budget=sp.budget, attn_scale=0.0, idx_scale=0.0, idx_rope_dim=8,
                idx_rope_theta=1e4)
    pos = np.arange(0, 512, 37)
    ref = orc.sequence(dims, case.k[0], case.v[0], case.kI[0], pos, case.q[0][pos],
                       case.qI[0][pos], case.w[0][pos], case.gate[0][pos], want_scores=True)
    dec = workloads.make_case("decode_32k_bf16", ctx=700, steps=2)
    d = dec.spec
    dims8 = dict(n_q_heads=d.n_q_heads, n_kv_heads=d.n_kv_heads, head_dim=d.head_dim,
                 n_idx_heads=d.n_idx_heads, idx_dim=d.idx_dim, block_size=d.block_size,
                 budget=d.budget, attn_scale=0.0, idx_scale=0.0)
    Kf, Vf = workloads.as_f32(dec.k[0]), workloads.as_f32(dec.v[0])
    Kc, Vc = orc.kv8_encode(Kf, True, 20.0), orc.kv8_encode(Vf, True, 20.0)
    r8 = orc.sequence_kv8(dims8, Kc, Vc, True, 0.05, 0.05, dec.kI[0], dec.q_pos[0], dec.q[0],
                          dec.qI[0], dec.w[0], dec.gate[0], want_scores=True)
    assert np.isfinite(ref["out"]).all() and np.isfinite(r8["out"]).all()
    print("ORACLE_ASAN_OK", flush=True)
""")

ABI_CHILD = textwrap.dedent("""
    import sys, ctypes as C
    sys.path.insert(0, ROOT)
    from block_sparse_attention_keys_amd import qsa
    L = qsa.lib(LIB)
    FAKE = 0x10000
    def P(**kw):
        base = dict(n_q_heads=16, n_kv_heads=2, head_dim=128, n_idx_heads=4, idx_dim=64,
                    block_size=64, budget=2048, dtype=qsa.QSA_BF16)
        base.update(kw)
        return qsa.make_params(**base)
    def B(**kw):
        base = dict(n_seqs=1, n_tokens=1, max_q_len=1, max_kv_len=100, kv_capacity=128,
                    page_size=0, max_pages=0, n_pages=0, cu_q=FAKE, past_len=FAKE,
                    page_table=None)
        base.update(kw)
        return qsa.qsa_batch(**base)
    bad_params = [dict(n_kv_heads=3), dict(head_dim=96), dict(block_size=48, ratio=48),
                  dict(budget=32), dict(idx_dim=48), dict(dtype=7), dict(kv_dtype=1),
                  dict(kv_dtype=qsa.QSA_KV_FP8, head_dim=64), dict(attn_scale=float("nan")),
                  dict(idx_rope_dim=3), dict(kv_rotate=1)]
    for kw in bad_params:
        ratio = kw.pop("ratio", None)
        p = qsa.make_params(**dict(dict(n_q_heads=16, n_kv_heads=2, head_dim=128, n_idx_heads=4,
                                        idx_dim=64, block_size=64, budget=2048,
                                        dtype=qsa.QSA_BF16), **kw), ratio=ratio)
        st = L.qsa_forward(C.byref(p), C.byref(B()), *([FAKE] * 15), 1 << 30, None)
        assert st != qsa.QSA_OK, kw
        assert len(L.qsa_last_error()) > 0
        assert L.qsa_workspace_size(C.byref(p), C.byref(B())) == 0
    for kw in [dict(n_seqs=0), dict(n_tokens=-1), dict(max_q_len=2), dict(kv_capacity=64),
               dict(cu_q=None), dict(page_table=FAKE),
               dict(page_size=64, max_pages=3, n_pages=3, kv_capacity=128, page_table=FAKE)]:
        assert L.qsa_forward(C.byref(P()), C.byref(B(**kw)), *([FAKE] * 15), 1 << 30,
                             None) != qsa.QSA_OK
    p, b = P(), B()
    assert L.qsa_forward(C.byref(p), C.byref(b), *([None] * 15), 1 << 30, None) == qsa.QSA_ERR_INVALID
    need = L.qsa_workspace_size(C.byref(p), C.byref(b))
    assert L.qsa_forward(C.byref(p), C.byref(b), *([FAKE] * 15), need - 1, None) == qsa.QSA_ERR_WORKSPACE
    big = B(n_tokens=8192, max_q_len=8192, max_kv_len=131072, kv_capacity=131072)
    assert L.qsa_workspace_size(C.byref(p), C.byref(big)) > 0
    assert L.qsa_forward_noalloc(C.byref(p), C.byref(big), *([FAKE] * 14), None) == qsa.QSA_ERR_WORKSPACE
    bp = qsa.make_block_params(2560, 64, 1e7, 1e-6)
    assert L.qsa_block_workspace_size(C.byref(p), C.byref(bp), C.byref(big)) > 0
    bp2 = qsa.make_block_params(100, 64, 1e7, 1e-6)
    assert L.qsa_block_forward(C.byref(p), C.byref(bp2), C.byref(b), *([FAKE] * 13), 1 << 30,
                               None) == qsa.QSA_ERR_INVALID
    assert L.qsa_pooled_ld(C.byref(p), C.byref(b)) > 0
    print("ABI_ASAN_OK", flush=True)
""")


def _run_child(code: str, lib: str, runtime: str) -> None:
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=23"
    env["OMP_NUM_THREADS"] = "2"
    prog = f"ROOT = {ROOT!r}\nLIB = {lib!r}\n" + code
    p = subprocess.run([sys.executable, "-c", prog], env=env, capture_output=True, text=True,
                       timeout=600)
    assert p.returncode == 0 and "ERROR: AddressSanitizer" not in p.stderr, (
        f"rc={p.returncode}\n{p.stdout[-2000:]}\n{p.stderr[-4000:]}")
    return p.stdout


@pytest.mark.slow
def test_oracle_under_host_asan():
    from oracle import build as ob
    lib = ob.build_asan()
    out = _run_child(ORACLE_CHILD, lib, ob.asan_runtime())
    assert "ORACLE_ASAN_OK" in out


@pytest.mark.slow
def test_abi_validation_under_host_asan():
    from block_sparse_attention_keys_amd import build as hb
    lib = hb.build_asan()
    out = _run_child(ABI_CHILD, lib, hb.asan_runtime())
    assert "ABI_ASAN_OK" in out
