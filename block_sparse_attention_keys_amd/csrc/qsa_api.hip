// C ABI of the QSA hot path: argument validation, workspace layout and launch
// sequencing.  No arithmetic of the method happens here; every step runs in
// the kernels of qsa_kernels.hip, qsa_prefill_ks.hip and qsa_block.hip (and,
// for the block's prefill-sized projections, hipBLASLt: qsa_blas.hip).  (The
// host fills only the rotary frequency tables, theta^(-2i/R) in fp64 with the
// C library's pow.)
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "qsa.h"
#include "qsa_internal.h"

// Device scratch of qsa_forward_noalloc: its workspace (scores, selections,
// split partials, key-stationary plan and partial states) for callers that
// cannot allocate.  Every GPU the library
// runs on holds one copy until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol):
// it uses the per-device address hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[QSA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

qsa_status fail(qsa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int64_t x) {
  int l = 0;
  while ((int64_t(1) << l) < x) ++l;
  return l;
}
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kAlign = 256;
constexpr int64_t kMfmaMinUnits = 512;  // (token, KV head) units that fill the chip without splits
constexpr int kMaxK = qsa::kPlanMaxK;

struct Plan {
  qsa::Geo geo;
  qsa::RopeTab idx_rope;  // pooled-key rotary frequencies
  qsa::AttnPlan attn;
  int elem;
  size_t off_scores, off_sel, off_nblk, off_part, total;
  // key-stationary prefill (attn.ks): entry lists, work items, partial states
  size_t off_ks_list, off_ks_items, off_ks_hist, off_ks_boff, off_ks_po, off_ks_pl, off_ks_qrot;
  int32_t ks_sub, max_q;
};

// Validates params/batch and derives every launch size from host values only.
qsa_status resolve(const qsa_params* P, const qsa_batch* Bt, Plan* out) {
  if (P == nullptr || Bt == nullptr) return fail(QSA_ERR_INVALID, "params or batch is NULL");
  const qsa_params& p = *P;
  const qsa_batch& b = *Bt;
  if (p.dtype != QSA_F32 && p.dtype != QSA_BF16)
    return fail(QSA_ERR_INVALID, "dtype %d is neither QSA_F32 nor QSA_BF16", p.dtype);
  if (p.n_q_heads <= 0 || p.n_kv_heads <= 0 || p.n_q_heads % p.n_kv_heads != 0)
    return fail(QSA_ERR_INVALID, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)",
                p.n_q_heads, p.n_kv_heads);
  const int G = p.n_q_heads / p.n_kv_heads;
  if (p.head_dim != 64 && p.head_dim != 128)
    return fail(QSA_ERR_UNSUPPORTED, "head_dim %d: supported 64, 128", p.head_dim);
  if (!qsa::attend_supported(G, p.head_dim))
    return fail(QSA_ERR_UNSUPPORTED, "n_q_heads/n_kv_heads = %d: supported 1, 2, 4, 8, 16", G);
  if (p.ratio != p.block_size)
    return fail(QSA_ERR_INVALID,
                "ratio (%d) must equal block_size (%d): the compression ratio is the block size",
                p.ratio, p.block_size);
  const int r = p.block_size;
  int k = 0;
  if (r != 0) {
    if (r < 0 || !is_pow2(r) || r < 4 || r > 256)
      return fail(QSA_ERR_UNSUPPORTED, "block_size %d: must be a power of two in [4, 256]", r);
    if (p.budget < r)
      return fail(QSA_ERR_INVALID, "budget (%d) must be >= block_size (%d)", p.budget, r);
    k = p.budget / r;
    if (k > kMaxK) return fail(QSA_ERR_UNSUPPORTED, "budget/block_size = %d exceeds %d", k, kMaxK);
    if (p.n_idx_heads < 1 || p.n_idx_heads > 16)
      return fail(QSA_ERR_UNSUPPORTED, "n_idx_heads %d: must be in [1, 16]", p.n_idx_heads);
    if (p.idx_dim != 32 && p.idx_dim != 64 && p.idx_dim != 128)
      return fail(QSA_ERR_UNSUPPORTED, "idx_dim %d: supported 32, 64, 128", p.idx_dim);
  }
  if (!(p.attn_scale == p.attn_scale) || !(p.idx_scale == p.idx_scale) || isinf(p.attn_scale) ||
      isinf(p.idx_scale))
    return fail(QSA_ERR_INVALID, "attn_scale / idx_scale must be finite");
  if (p.kv_dtype != QSA_KV_SAME && p.kv_dtype != QSA_KV_FP8)
    return fail(QSA_ERR_INVALID, "kv_dtype %d: QSA_KV_SAME (0) or QSA_KV_FP8 (2)", p.kv_dtype);
  if (p.kv_rotate != 0 && p.kv_rotate != 1)
    return fail(QSA_ERR_INVALID, "kv_rotate must be 0 or 1");
  if (p.kv_dtype == QSA_KV_FP8) {
    if (p.dtype != QSA_BF16 || p.head_dim != 128)
      return fail(QSA_ERR_UNSUPPORTED, "QSA_KV_FP8 needs dtype QSA_BF16 and head_dim 128");
    if (!(p.k_scale > 0.0f) || !(p.v_scale > 0.0f) || isinf(p.k_scale) || isinf(p.v_scale))
      return fail(QSA_ERR_INVALID, "k_scale and v_scale must be finite and > 0");
    if (p.kv_rotate && G < 4)
      return fail(QSA_ERR_UNSUPPORTED, "kv_rotate needs n_q_heads/n_kv_heads >= 4");
  } else if (p.kv_rotate) {
    return fail(QSA_ERR_INVALID, "kv_rotate needs kv_dtype QSA_KV_FP8");
  }
  if (p.idx_rope_dim != 0) {
    if (r == 0) return fail(QSA_ERR_INVALID, "idx_rope_dim must be 0 for a dense layer");
    if (p.idx_rope_dim < 0 || p.idx_rope_dim % 2 || p.idx_rope_dim > p.idx_dim)
      return fail(QSA_ERR_INVALID, "idx_rope_dim %d: an even number in [0, idx_dim]",
                  p.idx_rope_dim);
    if (!(p.idx_rope_theta > 0.0f) || isinf(p.idx_rope_theta))
      return fail(QSA_ERR_INVALID, "idx_rope_theta must be finite and > 0");
  }
  if (b.n_seqs < 1) return fail(QSA_ERR_INVALID, "n_seqs (%d) must be >= 1", b.n_seqs);
  if (b.n_tokens < 0) return fail(QSA_ERR_INVALID, "n_tokens (%d) must be >= 0", b.n_tokens);
  if (b.n_tokens > 0) {
    if (b.max_q_len < 1 || b.max_q_len > b.n_tokens)
      return fail(QSA_ERR_INVALID, "max_q_len (%d) must be in [1, n_tokens=%d]", b.max_q_len,
                  b.n_tokens);
    if (b.max_kv_len < 1 || b.max_kv_len < b.max_q_len)
      return fail(QSA_ERR_INVALID, "max_kv_len (%d) must be >= max_q_len (%d)", b.max_kv_len,
                  b.max_q_len);
    if (b.cu_q == nullptr || b.past_len == nullptr)
      return fail(QSA_ERR_INVALID, "cu_q and past_len must be device pointers");
  }
  if (b.kv_capacity < b.max_kv_len)
    return fail(QSA_ERR_INVALID, "kv_capacity (%d) < max_kv_len (%d)", b.kv_capacity,
                b.max_kv_len);
  if (b.page_size != 0) {
    if (!is_pow2(b.page_size))
      return fail(QSA_ERR_INVALID, "page_size %d must be a power of two", b.page_size);
    if (b.page_table == nullptr) return fail(QSA_ERR_INVALID, "paged layout needs page_table");
    if (b.max_pages < 1 || (int64_t)b.max_pages * b.page_size != b.kv_capacity)
      return fail(QSA_ERR_INVALID, "paged layout needs kv_capacity == max_pages * page_size");
    if (b.n_pages < 1) return fail(QSA_ERR_INVALID, "n_pages (%d) must be >= 1", b.n_pages);
  } else if (b.page_table != nullptr) {
    return fail(QSA_ERR_INVALID, "page_table given but page_size is 0");
  }

  Plan& pl = *out;
  qsa::Geo& g = pl.geo;
  pl.elem = p.dtype == QSA_BF16 ? qsa::kBF16 : qsa::kF32;
  g.Hq = p.n_q_heads;
  g.Hkv = p.n_kv_heads;
  g.G = G;
  g.D = p.head_dim;
  g.HI = r ? p.n_idx_heads : 0;
  g.dI = r ? p.idx_dim : 0;
  g.r = r;
  g.log2r = r ? ilog2(r) : 0;
  g.k = k;
  g.B = b.n_seqs;
  g.T = b.n_tokens;
  g.one_q = (b.n_tokens == b.n_seqs && b.max_q_len == 1) ? 1 : 0;
  g.cap = b.kv_capacity;
  g.page_size = b.page_size;
  g.log2ps = b.page_size ? ilog2(b.page_size) : 0;
  g.max_pages = b.max_pages;
  g.n_pages = b.n_pages;
  g.pooled_ld = r ? (int32_t)round_up((b.kv_capacity + r - 1) / r, 64) : 0;
  g.nbcap = r ? b.max_kv_len / r : 0;
  const double a_scale = p.attn_scale > 0.0f ? (double)p.attn_scale : 1.0 / sqrt((double)g.D);
  // Rotary indexer keys: frequencies theta^(-2i/R) in fp64 on the host.
  g.idx_rope_dim = p.idx_rope_dim;
  for (int i = 0; i < 64; ++i)
    out->idx_rope.f[i] = i < p.idx_rope_dim / 2
                        ? pow((double)p.idx_rope_theta, -2.0 * (double)i / (double)p.idx_rope_dim)
                        : 0.0;
  // 8-bit K/V: the K scale joins the softmax scale, and the rotated basis
  // multiplies every score by D (H H = D I); the V scale and the 1/D of the
  // un-rotation are applied to the output.
  g.kv8 = p.kv_dtype == QSA_KV_FP8 ? 1 : 0;
  g.rot = g.kv8 && p.kv_rotate ? 1 : 0;
  g.inv_k_scale = g.kv8 ? 1.0f / p.k_scale : 1.0f;
  g.inv_v_scale = g.kv8 ? 1.0f / p.v_scale : 1.0f;
  g.out_scale = g.kv8 ? (float)((double)p.v_scale / (g.rot ? (double)g.D : 1.0)) : 1.0f;
  g.attn_scale_log2 = (float)(a_scale * 1.4426950408889634 * (g.kv8 ? (double)p.k_scale : 1.0) /
                              (g.rot ? (double)g.D : 1.0));
  g.idx_scale = r ? (p.idx_scale > 0.0f ? p.idx_scale : (float)(1.0 / sqrt((double)g.dI))) : 0.0f;
  g.inv_r = r ? 1.0f / (float)r : 0.0f;
  g.cu_q = b.cu_q;
  g.past_len = b.past_len;
  g.page_table = b.page_table;

  // Split-KV plan.  A unit's list is cut into n_splits ranges of whole
  // 64-token tiles that differ by at most one tile.  The 4-wave decode kernel
  // aims at 512 workgroups (two per CU) with at least two tiles per split;
  // the one-wave generic kernel at 2048 waves.
  const int64_t max_list = r ? std::min<int64_t>(b.max_kv_len, (int64_t)k * r + r - 1)
                             : (int64_t)b.max_kv_len;
  const int64_t tiles = std::max<int64_t>(1, (max_list + 63) / 64);
  const int64_t units = std::max<int64_t>(1, (int64_t)b.n_tokens * g.Hkv);
  const int64_t waves = qsa::attend_waves(pl.elem, g.D);
  int64_t splits = waves > 1 ? std::min((512 + units - 1) / units, (tiles + 1) / 2)
                             : std::min((2048 + units - 1) / units, tiles);
  splits = std::max<int64_t>(1, std::min<int64_t>(splits, qsa::kPlanMaxSplits));
  pl.attn.n_splits = (int32_t)splits;
  pl.attn.tiles = (int32_t)tiles;
  // Many (token, KV head) units, as in prefill: the MFMA kernel, one wave per
  // unit.  Few units (decode): the split-list bandwidth kernels.
  pl.attn.mfma =
      (pl.elem == qsa::kBF16 && g.D == 128 && !g.kv8 && units >= kMfmaMinUnits) ? 1 : 0;
  // Long prefill chunks of a QSA layer: the key-stationary path, when its
  // entry packing and its plan's block table hold the call.
  pl.attn.ks = (r != 0 && b.max_q_len >= qsa::kKsMinQueries && qsa::ks_supported(g, pl.elem) &&
                g.nbcap + 1 <= qsa::kKsMaxBlocks && k + 1 <= qsa::kKsMaxSlots &&
                (int64_t)b.n_tokens < (int64_t(1) << 20) &&
                (int64_t)b.n_seqs * (g.nbcap + 2) <= (int64_t(1) << 16))
                   ? 1
                   : 0;
  if (pl.attn.ks) pl.attn.mfma = 0;
  if (pl.attn.mfma || pl.attn.ks) pl.attn.n_splits = 1;
  splits = pl.attn.n_splits;

  const int64_t T = b.n_tokens;
  size_t off = 0;
  pl.off_scores = off;
  off += round_up(T * std::max<int64_t>(g.nbcap, 1) * 4, kAlign);
  pl.off_sel = off;
  off += round_up(T * std::max(k, 1) * 4, kAlign);
  pl.off_nblk = off;
  off += round_up(T * 4, kAlign);
  pl.off_part = off;
  if (splits > 1) off += round_up(units * splits * G * (g.D + 2) * 4, kAlign);
  pl.ks_sub = (int32_t)std::min<int64_t>(std::max<int64_t>(T, 1), qsa::kKsSubTokens);
  pl.max_q = b.max_q_len;
  pl.off_ks_list = pl.off_ks_items = pl.off_ks_hist = pl.off_ks_boff = pl.off_ks_po =
      pl.off_ks_pl = pl.off_ks_qrot = off;
  if (pl.attn.ks) {
    const int64_t S = pl.ks_sub, k1 = k + 1;
    pl.off_ks_list = off;
    off += round_up(S * k1 * 4, kAlign);
    pl.off_ks_items = off;
    off += round_up(qsa::ks_item_bound(g, b.max_q_len, S) * 16, kAlign);
    pl.off_ks_hist = off;
    off += round_up((int64_t)b.n_seqs * qsa::ks_groups(b.max_q_len, S) * (g.nbcap + 1) * 4,
                    kAlign);
    pl.off_ks_boff = off;
    off += round_up((int64_t)b.n_seqs * (g.nbcap + 1) * 4, kAlign);
    pl.off_ks_po = off;
    off += round_up(S * g.Hq * k1 * g.D * 2, kAlign);
    pl.off_ks_pl = off;
    off += round_up(S * g.Hq * k1 * 4, kAlign);
    pl.off_ks_qrot = off;
    if (g.rot) off += round_up(S * g.Hq * g.D * 2, kAlign);
  }
  pl.total = T > 0 ? off : 0;
  if ((int64_t)g.T * g.Hkv > 0x7fffffff)
    return fail(QSA_ERR_UNSUPPORTED, "n_tokens * n_kv_heads exceeds the grid limit");
  // K/V cache rows are addressed by 32-bit row index inside the kernels.
  const int64_t kv_rows = b.page_size ? (int64_t)b.n_pages * g.Hkv * b.page_size
                                      : (int64_t)b.n_seqs * g.Hkv * b.kv_capacity;
  g.kv_esz = g.kv8 ? 1 : (pl.elem == qsa::kBF16 ? 2 : 4);
  if (kv_rows > 0x7fffffff)
    return fail(QSA_ERR_UNSUPPORTED, "the K/V cache holds more than 2^31 rows");
  return QSA_OK;
}

qsa_status check_ws(const Plan& pl, const void* ws, size_t ws_bytes) {
  if (pl.total == 0) return QSA_OK;
  if (ws == nullptr || ws_bytes < pl.total)
    return fail(QSA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                ws ? ws_bytes : (size_t)0, pl.total);
  if (!aligned(ws, 16)) return fail(QSA_ERR_INVALID, "workspace must be 16-byte aligned");
  return QSA_OK;
}

qsa_status need(const void* ptr, const char* name, size_t align) {
  if (ptr == nullptr) return fail(QSA_ERR_INVALID, "%s is NULL", name);
  if (!aligned(ptr, align)) return fail(QSA_ERR_INVALID, "%s is not %zu-byte aligned", name, align);
  return QSA_OK;
}

#define QSA_TRY(x)                  \
  do {                              \
    qsa_status _s = (x);            \
    if (_s != QSA_OK) return _s;    \
  } while (0)

qsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return QSA_OK;
  return fail(QSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

char* ws_at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// Attention over given selections: the key-stationary path or the others.
hipError_t attend_launch(const Plan& pl, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* sel, const int32_t* n_blocks, const void* gate, void* out,
                         void* ws, hipStream_t st) {
  if (pl.attn.ks) {
    qsa::KsWork w;
    w.list = reinterpret_cast<uint32_t*>(ws_at(ws, pl.off_ks_list));
    w.items = reinterpret_cast<int4*>(ws_at(ws, pl.off_ks_items));
    w.hist = reinterpret_cast<int32_t*>(ws_at(ws, pl.off_ks_hist));
    w.boff = reinterpret_cast<int32_t*>(ws_at(ws, pl.off_ks_boff));
    w.max_q = pl.max_q;
    w.po = reinterpret_cast<uint16_t*>(ws_at(ws, pl.off_ks_po));
    w.pl = reinterpret_cast<float*>(ws_at(ws, pl.off_ks_pl));
    w.qrot = reinterpret_cast<uint16_t*>(ws_at(ws, pl.off_ks_qrot));
    w.sub_tokens = pl.ks_sub;
    return qsa::launch_attend_ks(pl.geo, w, q, k_cache, v_cache, sel, n_blocks, gate, out, st);
  }
  float* part = reinterpret_cast<float*>(ws_at(ws, pl.off_part));
  return qsa::launch_attend(pl.geo, pl.elem, pl.attn, q, k_cache, v_cache, sel, n_blocks, gate,
                            out, part, st);
}

// Pointer checks of qsa_forward / qsa_forward_noalloc (everything but the workspace).
qsa_status check_forward_args(const Plan& pl, const void* q, const void* k_new,
                              const void* v_new, const void* q_idx, const void* k_idx_new,
                              const float* w, const void* gate, const void* k_cache,
                              const void* v_cache, const void* k_idx_cache, const float* pooled,
                              const void* out, const int32_t* sel_opt,
                              const int32_t* n_blocks_opt) {
  QSA_TRY(need(q, "q", 16));
  QSA_TRY(need(k_new, "k_new", 16));
  QSA_TRY(need(v_new, "v_new", 16));
  QSA_TRY(need(gate, "gate", 16));
  QSA_TRY(need(k_cache, "k_cache", 16));
  QSA_TRY(need(v_cache, "v_cache", 16));
  QSA_TRY(need(out, "out", 16));
  if (pl.geo.r != 0) {
    QSA_TRY(need(q_idx, "q_idx", 16));
    QSA_TRY(need(k_idx_new, "k_idx_new", 16));
    QSA_TRY(need(w, "w", 4));
    QSA_TRY(need(k_idx_cache, "k_idx_cache", 16));
    QSA_TRY(need(pooled, "pooled", 16));
    if (sel_opt) QSA_TRY(need(sel_opt, "sel", 4));
    if (n_blocks_opt) QSA_TRY(need(n_blocks_opt, "n_blocks", 4));
  }
  return QSA_OK;
}

// The scratch array's address on the current device, looked up once per
// device (each GPU holds its own copy of the array at its own address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

qsa_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(QSA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(QSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QSA_OK;
}

qsa_status forward_launch(const Plan& pl, const qsa_batch* batch, const void* q,
                          const void* k_new, const void* v_new, const void* q_idx,
                          const void* k_idx_new, const float* w, const void* gate,
                          void* k_cache, void* v_cache, void* k_idx_cache, float* pooled,
                          void* out, int32_t* sel_opt, int32_t* n_blocks_opt, void* ws,
                          hipStream_t st);

}  // namespace

extern "C" {

const char* qsa_last_error(void) { return g_last_error.c_str(); }

int64_t qsa_pooled_ld(const qsa_params* params, const qsa_batch* batch) {
  Plan pl;
  if (resolve(params, batch, &pl) != QSA_OK) return 0;
  return pl.geo.pooled_ld;
}

size_t qsa_workspace_size(const qsa_params* params, const qsa_batch* batch) {
  Plan pl;
  if (resolve(params, batch, &pl) != QSA_OK) return 0;
  return pl.total;
}

qsa_status qsa_store_kv(const qsa_params* params, const qsa_batch* batch, const void* k_new,
                        const void* v_new, void* k_cache, void* v_cache, void* stream) {
  g_last_error.clear();
  Plan pl;
  QSA_TRY(resolve(params, batch, &pl));
  if (batch->n_tokens == 0) return QSA_OK;
  QSA_TRY(need(k_new, "k_new", 16));
  QSA_TRY(need(v_new, "v_new", 16));
  QSA_TRY(need(k_cache, "k_cache", 16));
  QSA_TRY(need(v_cache, "v_cache", 16));
  return hip_status(qsa::launch_append_pool(pl.geo, pl.elem, k_new, v_new, nullptr, k_cache,
                                            v_cache, nullptr, nullptr, pl.idx_rope,
                                            static_cast<hipStream_t>(stream)),
                    "store launch");
}

qsa_status qsa_pool_keys(const qsa_params* params, const qsa_batch* batch,
                         const void* k_idx_new, void* k_idx_cache, float* pooled,
                         void* stream) {
  g_last_error.clear();
  Plan pl;
  QSA_TRY(resolve(params, batch, &pl));
  if (pl.geo.r == 0) return fail(QSA_ERR_INVALID, "dense layer (block_size 0) has no indexer");
  if (batch->n_tokens == 0) return QSA_OK;
  QSA_TRY(need(k_idx_new, "k_idx_new", 16));
  QSA_TRY(need(k_idx_cache, "k_idx_cache", 16));
  QSA_TRY(need(pooled, "pooled", 16));
  return hip_status(qsa::launch_append_pool(pl.geo, pl.elem, nullptr, nullptr, k_idx_new,
                                            nullptr, nullptr, k_idx_cache, pooled, pl.idx_rope,
                                            static_cast<hipStream_t>(stream)),
                    "qsa_pool_keys launch");
}

qsa_status qsa_score_select(const qsa_params* params, const qsa_batch* batch,
                            const void* q_idx, const float* w, const float* pooled,
                            int32_t* sel, int32_t* n_blocks, float* scores_opt, void* ws,
                            size_t ws_bytes, void* stream) {
  g_last_error.clear();
  Plan pl;
  QSA_TRY(resolve(params, batch, &pl));
  if (pl.geo.r == 0) return fail(QSA_ERR_INVALID, "dense layer (block_size 0) has no indexer");
  if (batch->n_tokens == 0) return QSA_OK;
  QSA_TRY(need(q_idx, "q_idx", 16));
  QSA_TRY(need(w, "w", 4));
  QSA_TRY(need(pooled, "pooled", 16));
  QSA_TRY(need(sel, "sel", 4));
  QSA_TRY(need(n_blocks, "n_blocks", 4));
  if (scores_opt != nullptr) QSA_TRY(need(scores_opt, "scores", 4));
  QSA_TRY(check_ws(pl, ws, ws_bytes));
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* scores = scores_opt ? scores_opt : reinterpret_cast<float*>(ws_at(ws, pl.off_scores));
  QSA_TRY(hip_status(qsa::launch_score(pl.geo, pl.elem, q_idx, w, const_cast<float*>(pooled),
                                       scores, st),
                     "score launch"));
  return hip_status(qsa::launch_select(pl.geo, scores, sel, n_blocks, st), "select launch");
}

qsa_status qsa_attend(const qsa_params* params, const qsa_batch* batch, const void* q,
                      const void* k_cache, const void* v_cache, const int32_t* sel,
                      const int32_t* n_blocks, const void* gate, void* out, void* ws,
                      size_t ws_bytes, void* stream) {
  g_last_error.clear();
  Plan pl;
  QSA_TRY(resolve(params, batch, &pl));
  if (batch->n_tokens == 0) return QSA_OK;
  QSA_TRY(need(q, "q", 16));
  QSA_TRY(need(k_cache, "k_cache", 16));
  QSA_TRY(need(v_cache, "v_cache", 16));
  QSA_TRY(need(gate, "gate", 16));
  QSA_TRY(need(out, "out", 16));
  if (pl.geo.r != 0) {
    QSA_TRY(need(sel, "sel", 4));
    QSA_TRY(need(n_blocks, "n_blocks", 4));
  }
  QSA_TRY(check_ws(pl, ws, ws_bytes));
  return hip_status(attend_launch(pl, q, k_cache, v_cache, sel, n_blocks, gate, out, ws,
                                  static_cast<hipStream_t>(stream)),
                    "attend launch");
}

qsa_status qsa_forward(const qsa_params* params, const qsa_batch* batch, const void* q,
                       const void* k_new, const void* v_new, const void* q_idx,
                       const void* k_idx_new, const float* w, const void* gate,
                       void* k_cache, void* v_cache, void* k_idx_cache, float* pooled,
                       void* out, int32_t* sel_opt, int32_t* n_blocks_opt, void* ws,
                       size_t ws_bytes, void* stream) {
  g_last_error.clear();
  Plan pl;
  QSA_TRY(resolve(params, batch, &pl));
  if (batch->n_tokens == 0) return QSA_OK;
  QSA_TRY(check_forward_args(pl, q, k_new, v_new, q_idx, k_idx_new, w, gate, k_cache, v_cache,
                             k_idx_cache, pooled, out, sel_opt, n_blocks_opt));
  QSA_TRY(check_ws(pl, ws, ws_bytes));
  return forward_launch(pl, batch, q, k_new, v_new, q_idx, k_idx_new, w, gate, k_cache, v_cache,
                        k_idx_cache, pooled, out, sel_opt, n_blocks_opt, ws,
                        static_cast<hipStream_t>(stream));
}

qsa_status qsa_forward_noalloc(const qsa_params* params, const qsa_batch* batch, const void* q,
                               const void* k_new, const void* v_new, const void* q_idx,
                               const void* k_idx_new, const float* w, const void* gate,
                               void* k_cache, void* v_cache, void* k_idx_cache, float* pooled,
                               void* out, int32_t* sel_opt, int32_t* n_blocks_opt,
                               void* stream) {
  g_last_error.clear();
  Plan pl;
  QSA_TRY(resolve(params, batch, &pl));
  if (batch->n_tokens == 0) return QSA_OK;
  QSA_TRY(check_forward_args(pl, q, k_new, v_new, q_idx, k_idx_new, w, gate, k_cache, v_cache,
                             k_idx_cache, pooled, out, sel_opt, n_blocks_opt));
  if (pl.total > (size_t)QSA_NOALLOC_SCRATCH_BYTES)
    return fail(QSA_ERR_WORKSPACE,
                "this call needs %zu bytes of workspace; qsa_forward_noalloc holds %zu "
                "(use qsa_forward with a workspace, or split the batch)",
                pl.total, (size_t)QSA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  QSA_TRY(scratch_on_current_device(&ws));
  return forward_launch(pl, batch, q, k_new, v_new, q_idx, k_idx_new, w, gate, k_cache, v_cache,
                        k_idx_cache, pooled, out, sel_opt, n_blocks_opt, ws,
                        static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// The launch sequence of one QSA layer step (arguments already validated).
qsa_status forward_launch(const Plan& pl, const qsa_batch* batch, const void* q,
                          const void* k_new, const void* v_new, const void* q_idx,
                          const void* k_idx_new, const float* w, const void* gate,
                          void* k_cache, void* v_cache, void* k_idx_cache, float* pooled,
                          void* out, int32_t* sel_opt, int32_t* n_blocks_opt, void* ws,
                          hipStream_t st) {
  const bool qsa_layer = pl.geo.r != 0;
  int32_t* sel = sel_opt ? sel_opt : reinterpret_cast<int32_t*>(ws_at(ws, pl.off_sel));
  int32_t* nblk = n_blocks_opt ? n_blocks_opt : reinterpret_cast<int32_t*>(ws_at(ws, pl.off_nblk));
  if (qsa_layer && batch->max_q_len == 1) {
    // Decode form: one launch appends, pools and scores.
    float* scores = reinterpret_cast<float*>(ws_at(ws, pl.off_scores));
    const qsa::AppendArgs ap = {k_new, v_new, k_idx_new, k_cache, v_cache, k_idx_cache};
    QSA_TRY(hip_status(
        qsa::launch_score_append(pl.geo, pl.elem, q_idx, w, pooled, scores, ap, pl.idx_rope, st),
        "append/score launch"));
  } else {
    QSA_TRY(hip_status(qsa::launch_append_pool(pl.geo, pl.elem, k_new, v_new,
                                               qsa_layer ? k_idx_new : nullptr, k_cache, v_cache,
                                               qsa_layer ? k_idx_cache : nullptr,
                                               qsa_layer ? pooled : nullptr, pl.idx_rope, st),
                       "append/pool launch"));
    if (qsa_layer) {
      float* scores = reinterpret_cast<float*>(ws_at(ws, pl.off_scores));
      QSA_TRY(hip_status(qsa::launch_score(pl.geo, pl.elem, q_idx, w, pooled, scores, st),
                         "score launch"));
    }
  }
  // Decode attention with few candidate blocks makes the selection itself
  // (no separate select launch); otherwise select, then attend.
  const bool fused = qsa_layer && !pl.attn.mfma && !pl.attn.ks && pl.elem == qsa::kBF16 &&
                     pl.geo.D == 128 && pl.geo.nbcap <= qsa::kSelectInKernelMaxBlocks;
  float* part = reinterpret_cast<float*>(ws_at(ws, pl.off_part));
  if (fused) {
    const qsa::InKernelSelect fs = {reinterpret_cast<const float*>(ws_at(ws, pl.off_scores)), sel,
                                    nblk};
    return hip_status(qsa::launch_attend(pl.geo, pl.elem, pl.attn, q, k_cache, v_cache, nullptr,
                                         nullptr, gate, out, part, st, fs),
                      "attend launch");
  }
  if (qsa_layer) {
    float* scores = reinterpret_cast<float*>(ws_at(ws, pl.off_scores));
    QSA_TRY(hip_status(qsa::launch_select(pl.geo, scores, sel, nblk, st), "select launch"));
  }
  return hip_status(attend_launch(pl, q, k_cache, v_cache, sel, nblk, gate, out, ws, st),
                    "attend launch");
}

}  // namespace

// ---------------------------------------------------------------------------
// The block front end.
namespace {

struct BlockPlan {
  Plan core;
  int n_in, d_model, hqd, S1, S2;
  size_t off_p1, off_q, off_gate, off_k, off_v, off_qI, off_kI, off_w, off_attn, off_p2,
      off_core, total;
};

qsa_status resolve_block(const qsa_params* P, const qsa_block_params* BP, const qsa_batch* Bt,
                         BlockPlan* out) {
  QSA_TRY(resolve(P, Bt, &out->core));
  if (BP == nullptr) return fail(QSA_ERR_INVALID, "block params are NULL");
  const qsa_params& p = *P;
  const qsa_block_params& bp = *BP;
  if (p.dtype != QSA_BF16) return fail(QSA_ERR_UNSUPPORTED, "the block needs dtype QSA_BF16");
  if (bp.d_model <= 0 || bp.d_model % 32 != 0 || bp.d_model > 65536)
    return fail(QSA_ERR_INVALID, "d_model %d: a positive multiple of 32, at most 65536",
                bp.d_model);
  if (bp.rotary_dim < 0 || bp.rotary_dim % 2 || bp.rotary_dim > p.head_dim)
    return fail(QSA_ERR_INVALID, "rotary_dim %d: an even number in [0, head_dim]", bp.rotary_dim);
  if (bp.rotary_dim > 0 && (!(bp.rope_theta > 0.0f) || isinf(bp.rope_theta)))
    return fail(QSA_ERR_INVALID, "rope_theta must be finite and > 0");
  if (!(bp.norm_eps >= 0.0f) || isinf(bp.norm_eps))
    return fail(QSA_ERR_INVALID, "norm_eps must be finite and >= 0");
  const qsa::Geo& g = out->core.geo;
  const int64_t T = Bt->n_tokens;
  const int64_t hqd = (int64_t)g.Hq * g.D, hkvd = (int64_t)g.Hkv * g.D;
  const int64_t n_in = 2 * hqd + 2 * hkvd + (g.r ? (int64_t)g.HI * g.dI + g.dI : 0);
  const int64_t lim = int64_t(1) << 31;  // operand bytes the GEMM addresses
  if (T * bp.d_model * 2 >= lim || n_in * bp.d_model * 2 >= lim || hqd * bp.d_model * 2 >= lim ||
      T * hqd * 2 >= lim)
    return fail(QSA_ERR_UNSUPPORTED, "a projection operand reaches 2 GiB");
  out->n_in = (int)n_in;
  out->d_model = bp.d_model;
  out->hqd = (int)hqd;
  out->S1 = T > 0 ? qsa::gemm_splits((int)T, (int)n_in, bp.d_model) : 1;
  out->S2 = T > 0 ? qsa::gemm_splits((int)T, bp.d_model, (int)hqd) : 1;
  size_t off = 0;
  auto take = [&](int64_t bytes) {
    const size_t o = off;
    off += round_up(std::max<int64_t>(bytes, 1), kAlign);
    return o;
  };
  out->off_p1 = take(out->S1 * T * n_in * 4);
  out->off_q = take(T * hqd * 2);
  out->off_gate = take(T * hqd * 2);
  out->off_k = take(T * hkvd * 2);
  out->off_v = take(T * hkvd * 2);
  out->off_qI = take(T * g.HI * g.dI * 2);
  out->off_kI = take(T * g.dI * 2);
  out->off_w = take(T * g.HI * 4);
  out->off_attn = take(T * hqd * 2);
  out->off_p2 = take(out->S2 * T * bp.d_model * 4);
  out->off_core = take((int64_t)out->core.total);
  out->total = T > 0 ? off : 0;
  return QSA_OK;
}

}  // namespace

extern "C" {

size_t qsa_block_workspace_size(const qsa_params* params, const qsa_block_params* block,
                                const qsa_batch* batch) {
  BlockPlan bl;
  if (resolve_block(params, block, batch, &bl) != QSA_OK) return 0;
  return bl.total;
}

qsa_status qsa_block_forward(const qsa_params* params, const qsa_block_params* block,
                             const qsa_batch* batch, const void* x, const void* w_in,
                             const void* q_norm, const void* k_norm, const void* w_o,
                             void* k_cache, void* v_cache, void* k_idx_cache, float* pooled,
                             void* y, int32_t* sel_opt, int32_t* n_blocks_opt, void* ws,
                             size_t ws_bytes, void* stream) {
  g_last_error.clear();
  BlockPlan bl;
  QSA_TRY(resolve_block(params, block, batch, &bl));
  if (batch->n_tokens == 0) return QSA_OK;
  QSA_TRY(need(x, "x", 16));
  QSA_TRY(need(w_in, "w_in", 16));
  QSA_TRY(need(q_norm, "q_norm", 2));
  QSA_TRY(need(k_norm, "k_norm", 2));
  QSA_TRY(need(w_o, "w_o", 16));
  QSA_TRY(need(k_cache, "k_cache", 16));
  QSA_TRY(need(v_cache, "v_cache", 16));
  QSA_TRY(need(y, "y", 16));
  const qsa::Geo& g = bl.core.geo;
  if (g.r != 0) {
    QSA_TRY(need(k_idx_cache, "k_idx_cache", 16));
    QSA_TRY(need(pooled, "pooled", 16));
    if (sel_opt) QSA_TRY(need(sel_opt, "sel", 4));
    if (n_blocks_opt) QSA_TRY(need(n_blocks_opt, "n_blocks", 4));
  }
  if (ws == nullptr || ws_bytes < bl.total)
    return fail(QSA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                ws ? ws_bytes : (size_t)0, bl.total);
  if (!aligned(ws, 16)) return fail(QSA_ERR_INVALID, "workspace must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int T = batch->n_tokens;
  float* p1 = reinterpret_cast<float*>(ws_at(ws, bl.off_p1));
  QSA_TRY(hip_status(
      qsa::launch_proj_gemm(x, w_in, p1, nullptr, T, bl.n_in, bl.d_model, bl.S1, st),
      "input projection launch"));
  qsa::BlockPrepArgs a;
  a.part = p1;
  a.S = bl.S1;
  a.n_in = bl.n_in;
  a.eps = block->norm_eps;
  a.rotary_dim = block->rotary_dim;
  for (int i = 0; i < 64; ++i) a.idx_freq[i] = bl.core.idx_rope.f[i];
  for (int i = 0; i < 64; ++i)
    a.freq[i] = i < block->rotary_dim / 2
                    ? pow((double)block->rope_theta, -2.0 * (double)i / (double)block->rotary_dim)
                    : 0.0;
  a.q_norm = static_cast<const uint16_t*>(q_norm);
  a.k_norm = static_cast<const uint16_t*>(k_norm);
  a.q = reinterpret_cast<uint16_t*>(ws_at(ws, bl.off_q));
  a.gate = reinterpret_cast<uint16_t*>(ws_at(ws, bl.off_gate));
  a.k = reinterpret_cast<uint16_t*>(ws_at(ws, bl.off_k));
  a.v = reinterpret_cast<uint16_t*>(ws_at(ws, bl.off_v));
  a.q_idx = reinterpret_cast<uint16_t*>(ws_at(ws, bl.off_qI));
  a.k_idx = reinterpret_cast<uint16_t*>(ws_at(ws, bl.off_kI));
  a.w = reinterpret_cast<float*>(ws_at(ws, bl.off_w));
  QSA_TRY(hip_status(qsa::launch_block_prep(g, a, st), "block prep launch"));
  void* attn = ws_at(ws, bl.off_attn);
  QSA_TRY(forward_launch(bl.core, batch, a.q, a.k, a.v, g.r ? a.q_idx : nullptr,
                         g.r ? a.k_idx : nullptr, g.r ? a.w : nullptr, a.gate, k_cache, v_cache,
                         k_idx_cache, pooled, attn, sel_opt, n_blocks_opt,
                         ws_at(ws, bl.off_core), st));
  float* p2 = reinterpret_cast<float*>(ws_at(ws, bl.off_p2));
  QSA_TRY(hip_status(qsa::launch_proj_gemm(attn, w_o, p2, y, T, bl.d_model, bl.hqd, bl.S2, st),
                     "output projection launch"));
  if (bl.S2 == 1) return QSA_OK;  // the GEMM wrote y
  return hip_status(qsa::launch_proj_reduce(p2, bl.S2, (int64_t)T * bl.d_model, y, st),
                    "output reduce launch");
}

#ifdef QSA_COUNT_KEYS
// Debug builds only (include/qsa_probe.h).
int64_t qsa_probe_keys_visited(int32_t reset) {
  unsigned long long v = 0, w = 0;
  if (qsa::keys_visited(&v, reset != 0) != hipSuccess) return -1;
  if (qsa::ks_keys_visited(&w, reset != 0) != hipSuccess) return -1;
  return (int64_t)(v + w);
}

void qsa_probe_library_gemm(int32_t enable) { qsa::lt_set_enabled(enable != 0); }

int32_t qsa_probe_gemm(const void* A, const void* B, void* D, int32_t d_f32, int32_t M, int32_t N,
                       int32_t K, void* stream) {
  if (A == nullptr || B == nullptr || D == nullptr || M <= 0 || N <= 0 || K <= 0) return -1;
  const hipError_t e = qsa::lt_gemm(A, B, D, d_f32 != 0, M, N, K, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : (e == hipErrorNotSupported ? 1 : -1);
}
#endif

}  // extern "C"

