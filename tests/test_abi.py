"""The C ABI on the CPU: the library loads, exports every function that
include/qsa.h declares, and rejects bad arguments before launching anything
(no GPU is touched: every call here fails validation or is a no-op)."""
import ctypes as C
import os
import re

import pytest

from block_sparse_attention_keys_amd import qsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(qsa.LIB_PATH):
        from block_sparse_attention_keys_amd import build
        build.build()
    return qsa.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("qsa_pool_keys", "qsa_score_select", "qsa_attend", "qsa_forward",
              "qsa_workspace_size", "qsa_last_error", "qsa_pooled_ld"):
        assert n in names
    assert sorted(qsa.EXPORTS) == names


def test_every_declared_symbol_is_exported(L):
    for n in declared_functions():
        assert hasattr(L, n), n


def test_binding_argument_counts_match_header(L):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for name in declared_functions():
        m = re.search(name + r"\s*\(([^)]*)\)", text)
        params = [q for q in m.group(1).split(",") if q.strip() and q.strip() != "void"]
        assert len(getattr(L, name).argtypes) == len(params), name


def test_struct_layouts_match_header():
    # field order and sizes of the ctypes mirrors against the header text
    text = open(HEADER).read()
    body = text[text.index("typedef struct {"):text.index("} qsa_params;")]
    fields = re.findall(r"(int32_t|float)\s+(\w+);", body)
    assert [f for _, f in fields] == [f for f, _ in qsa.qsa_params._fields_]
    assert C.sizeof(qsa.qsa_params) == 4 * len(fields)
    body = text[text.index("} qsa_params;"):text.index("} qsa_batch;")]
    names = re.findall(r"(?:int32_t|const int32_t\s*\*)\s*(\w+);", body)
    assert names == [f for f, _ in qsa.qsa_batch._fields_]


def test_block_struct_layout_matches_header():
    text = open(HEADER).read()
    i = text.index("} qsa_batch;")
    body = text[text.index("typedef struct {", i):text.index("} qsa_block_params;")]
    fields = re.findall(r"(int32_t|float)\s+(\w+);", body)
    assert [f for _, f in fields] == [f for f, _ in qsa.qsa_block_params._fields_]
    assert C.sizeof(qsa.qsa_block_params) == 4 * len(fields)


def P(**kw):
    base = dict(n_q_heads=16, n_kv_heads=2, head_dim=128, n_idx_heads=4, idx_dim=64,
                block_size=64, budget=2048, dtype=qsa.QSA_BF16)
    base.update(kw)
    ratio = base.pop("ratio", None)
    return qsa.make_params(ratio=ratio, **base)


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def Bt(**kw):
    base = dict(n_seqs=1, n_tokens=1, max_q_len=1, max_kv_len=100, kv_capacity=128,
                page_size=0, max_pages=0, n_pages=0, cu_q=FAKE, past_len=FAKE, page_table=None)
    base.update(kw)
    return qsa.qsa_batch(**base)


def fwd(L, p, b, ptr=FAKE, ws_bytes=1 << 30):
    return L.qsa_forward(C.byref(p), C.byref(b), *([ptr] * 15), ws_bytes, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(n_kv_heads=3), qsa.QSA_ERR_INVALID, "multiple"),
    (dict(n_q_heads=0), qsa.QSA_ERR_INVALID, "multiple"),
    (dict(head_dim=96), qsa.QSA_ERR_UNSUPPORTED, "head_dim"),
    (dict(n_q_heads=64, n_kv_heads=2), qsa.QSA_ERR_UNSUPPORTED, "n_q_heads/n_kv_heads"),
    (dict(ratio=32), qsa.QSA_ERR_INVALID, "ratio"),
    (dict(block_size=48, ratio=48), qsa.QSA_ERR_UNSUPPORTED, "power of two"),
    (dict(block_size=2, ratio=2), qsa.QSA_ERR_UNSUPPORTED, "power of two"),
    (dict(budget=32), qsa.QSA_ERR_INVALID, "budget"),
    (dict(budget=64 * 4096), qsa.QSA_ERR_UNSUPPORTED, "exceeds"),
    (dict(n_idx_heads=0), qsa.QSA_ERR_UNSUPPORTED, "n_idx_heads"),
    (dict(idx_dim=48), qsa.QSA_ERR_UNSUPPORTED, "idx_dim"),
    (dict(dtype=7), qsa.QSA_ERR_INVALID, "dtype"),
    (dict(attn_scale=float("nan")), qsa.QSA_ERR_INVALID, "finite"),
    (dict(kv_dtype=1), qsa.QSA_ERR_INVALID, "kv_dtype"),
    (dict(kv_dtype=qsa.QSA_KV_FP8, kv_rotate=2), qsa.QSA_ERR_INVALID, "kv_rotate"),
    (dict(kv_rotate=1), qsa.QSA_ERR_INVALID, "needs kv_dtype"),
    (dict(kv_dtype=qsa.QSA_KV_FP8, dtype=qsa.QSA_F32), qsa.QSA_ERR_UNSUPPORTED, "QSA_KV_FP8"),
    (dict(kv_dtype=qsa.QSA_KV_FP8, head_dim=64), qsa.QSA_ERR_UNSUPPORTED, "QSA_KV_FP8"),
    (dict(kv_dtype=qsa.QSA_KV_FP8, k_scale=0.0), qsa.QSA_ERR_INVALID, "k_scale"),
    (dict(kv_dtype=qsa.QSA_KV_FP8, v_scale=float("inf")), qsa.QSA_ERR_INVALID, "k_scale"),
    (dict(kv_dtype=qsa.QSA_KV_FP8, kv_rotate=1, n_q_heads=4), qsa.QSA_ERR_UNSUPPORTED,
     "kv_rotate"),
])
def test_params_rejected(L, kw, status, needle):
    assert fwd(L, P(**kw), Bt()) == status
    assert needle in qsa.last_error()
    assert qsa.qsa_workspace_size(P(**kw), Bt()) == 0


@pytest.mark.parametrize("kw,status,needle", [
    (dict(n_seqs=0), qsa.QSA_ERR_INVALID, "n_seqs"),
    (dict(n_tokens=-1), qsa.QSA_ERR_INVALID, "n_tokens"),
    (dict(max_q_len=2), qsa.QSA_ERR_INVALID, "max_q_len"),
    (dict(kv_capacity=64), qsa.QSA_ERR_INVALID, "kv_capacity"),
    (dict(cu_q=None), qsa.QSA_ERR_INVALID, "cu_q"),
    (dict(page_size=48, max_pages=3, n_pages=3, kv_capacity=144, page_table=FAKE),
     qsa.QSA_ERR_INVALID, "power of two"),
    (dict(page_size=64, max_pages=2, n_pages=2, kv_capacity=128), qsa.QSA_ERR_INVALID,
     "page_table"),
    (dict(page_size=64, max_pages=3, n_pages=3, kv_capacity=128, page_table=FAKE),
     qsa.QSA_ERR_INVALID, "max_pages"),
    (dict(page_table=FAKE), qsa.QSA_ERR_INVALID, "page_size is 0"),
])
def test_batch_rejected(L, kw, status, needle):
    assert fwd(L, P(), Bt(**kw)) == status
    assert needle in qsa.last_error()


def test_null_and_misaligned_pointers(L):
    p, b = P(), Bt()
    assert fwd(L, p, b, ptr=None) == qsa.QSA_ERR_INVALID
    assert "NULL" in qsa.last_error()
    assert fwd(L, p, b, ptr=FAKE + 2) == qsa.QSA_ERR_INVALID
    assert "aligned" in qsa.last_error()


def test_workspace_checked(L):
    p, b = P(), Bt()
    need = qsa.qsa_workspace_size(p, b)
    assert need > 0
    assert fwd(L, p, b, ws_bytes=need - 1) == qsa.QSA_ERR_WORKSPACE
    assert "workspace" in qsa.last_error()


def test_zero_tokens_is_a_noop(L):
    b = Bt(n_tokens=0, cu_q=None, past_len=None)
    assert qsa.qsa_workspace_size(P(), b) == 0
    assert fwd(L, P(), b, ptr=None, ws_bytes=0) == qsa.QSA_OK
    assert L.qsa_attend(C.byref(P()), C.byref(b), *([None] * 8), 0, None) == qsa.QSA_OK


def test_store_kv_validates(L):
    p = P(kv_dtype=qsa.QSA_KV_FP8)
    assert L.qsa_store_kv(C.byref(p), C.byref(Bt()), FAKE, None, FAKE, FAKE, None) == \
        qsa.QSA_ERR_INVALID
    assert "v_new" in qsa.last_error()
    assert L.qsa_store_kv(C.byref(P(kv_rotate=1)), C.byref(Bt()), FAKE, FAKE, FAKE, FAKE,
                          None) == qsa.QSA_ERR_INVALID
    b = Bt(n_tokens=0, cu_q=None, past_len=None)
    assert L.qsa_store_kv(C.byref(p), C.byref(b), None, None, None, None, None) == qsa.QSA_OK


@pytest.mark.parametrize("kw,bkw,status,needle", [
    (dict(), dict(d_model=100), qsa.QSA_ERR_INVALID, "d_model"),
    (dict(), dict(rotary_dim=130), qsa.QSA_ERR_INVALID, "rotary_dim"),
    (dict(), dict(rotary_dim=7), qsa.QSA_ERR_INVALID, "rotary_dim"),
    (dict(), dict(rope_theta=0.0), qsa.QSA_ERR_INVALID, "rope_theta"),
    (dict(), dict(norm_eps=-1.0), qsa.QSA_ERR_INVALID, "norm_eps"),
    (dict(dtype=qsa.QSA_F32), dict(), qsa.QSA_ERR_UNSUPPORTED, "QSA_BF16"),
    (dict(idx_rope_dim=66), dict(), qsa.QSA_ERR_INVALID, "idx_rope_dim"),
    (dict(idx_rope_dim=32, idx_rope_theta=0.0), dict(), qsa.QSA_ERR_INVALID, "idx_rope_theta"),
    (dict(block_size=0, ratio=0, idx_rope_dim=32, idx_rope_theta=1e4), dict(),
     qsa.QSA_ERR_INVALID, "dense"),
])
def test_block_params_rejected(L, kw, bkw, status, needle):
    base = dict(d_model=512, rotary_dim=64, rope_theta=1e6, norm_eps=1e-6)
    base.update(bkw)
    bp = qsa.make_block_params(**base)
    p = P(**kw)
    rc = L.qsa_block_forward(C.byref(p), C.byref(bp), C.byref(Bt()), *([FAKE] * 13), 1 << 30, None)
    assert rc == status
    assert needle in qsa.last_error()
    assert qsa.qsa_block_workspace_size(p, bp, Bt()) == 0


def test_block_zero_tokens_is_a_noop(L):
    p, bp = P(), qsa.make_block_params(512, 64, 1e6)
    b = Bt(n_tokens=0, cu_q=None, past_len=None)
    assert qsa.qsa_block_workspace_size(p, bp, b) == 0
    assert L.qsa_block_forward(C.byref(p), C.byref(bp), C.byref(b), *([None] * 13), 0,
                               None) == qsa.QSA_OK


def test_block_workspace_and_pointers(L):
    p, bp = P(idx_rope_dim=64, idx_rope_theta=1e6), qsa.make_block_params(512, 64, 1e6)
    need = qsa.qsa_block_workspace_size(p, bp, Bt())
    assert need > qsa.qsa_workspace_size(p, Bt()) > 0
    args = [FAKE] * 13
    assert L.qsa_block_forward(C.byref(p), C.byref(bp), C.byref(Bt()), *args, need - 1,
                               None) == qsa.QSA_ERR_WORKSPACE
    args[0] = None
    assert L.qsa_block_forward(C.byref(p), C.byref(bp), C.byref(Bt()), *args, need,
                               None) == qsa.QSA_ERR_INVALID
    assert "x is NULL" in qsa.last_error()


def test_dense_layer_rejects_indexer_calls(L):
    p = P(block_size=0, ratio=0)
    assert L.qsa_pool_keys(C.byref(p), C.byref(Bt()), FAKE, FAKE, FAKE, None) == qsa.QSA_ERR_INVALID
    assert "dense" in qsa.last_error()


def test_pooled_ld(L):
    assert qsa.qsa_pooled_ld(P(), Bt(kv_capacity=32768 + 64, max_kv_len=32769)) == 576
    assert qsa.qsa_pooled_ld(P(block_size=128, ratio=128), Bt(kv_capacity=262272,
                                                              max_kv_len=262272)) == 2112
    assert qsa.qsa_pooled_ld(P(block_size=0, ratio=0), Bt()) == 0


def test_workspace_grows_with_batch(L):
    small = qsa.qsa_workspace_size(P(), Bt())
    big = qsa.qsa_workspace_size(P(), Bt(n_tokens=64, max_q_len=64, max_kv_len=4096,
                                         kv_capacity=4096))
    assert big > small > 0


PROBE_HEADER = os.path.join(ROOT, "include", "qsa_probe.h")


def test_probe_symbols_only_in_the_probe_build(L):
    """include/qsa_probe.h: the row counter, the GEMM-library switch and the
    direct library product exist in libqsa_probe.so only; the probe build
    exports the whole boundary as well."""
    if not os.path.exists(qsa.PROBE_PATH):
        from block_sparse_attention_keys_amd import build
        build.build(build.PROBE_LIB, build.PROBE_FLAGS)
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    probe_names = sorted(set(re.findall(r"\b(qsa_[a-z_]+)\s*\(", text)))
    assert probe_names == ["qsa_probe_gemm", "qsa_probe_keys_visited", "qsa_probe_library_gemm"]
    P = C.CDLL(qsa.PROBE_PATH)
    for n in probe_names:
        assert hasattr(P, n), n
        assert not hasattr(L, n), f"{n} leaked into the product library"
    for n in declared_functions():
        assert hasattr(P, n), n


def test_noalloc_entry_validates_before_touching_the_gpu(L):
    """qsa_forward_noalloc: the same argument checks as qsa_forward, and a call
    whose workspace exceeds the library's scratch is rejected before any HIP
    call (nothing here has a GPU)."""
    def call(p, b, ptr=FAKE):
        return L.qsa_forward_noalloc(C.byref(p), C.byref(b), *([ptr] * 14), None)

    assert call(P(n_kv_heads=3), Bt()) == qsa.QSA_ERR_INVALID
    assert call(P(), Bt(), ptr=FAKE + 2) == qsa.QSA_ERR_INVALID
    assert "aligned" in qsa.last_error()
    big = Bt(n_tokens=8192, max_q_len=8192, max_kv_len=131072, kv_capacity=131072)
    assert qsa.qsa_workspace_size(P(), big) > qsa.QSA_NOALLOC_SCRATCH_BYTES
    assert call(P(), big) == qsa.QSA_ERR_WORKSPACE
    assert "qsa_forward_noalloc holds" in qsa.last_error()
    b0 = Bt(n_tokens=0, cu_q=None, past_len=None)
    assert call(P(), b0, ptr=None) == qsa.QSA_OK
