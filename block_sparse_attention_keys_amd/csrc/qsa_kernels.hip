// QSA hot-path kernels for gfx950 (MI355X): wave64, LDS, dot2 / MFMA.
//
// Kernels (one QSA layer step):
//   append_pool   write new K/V/indexer-key rows at each sequence's past_len and
//                 pool every block the new tokens complete (mean of r indexer
//                 keys, fp32, tokens ascending), pooling in workgroups of its
//                 own dispatched ahead of the copies.
//   score         relu-weighted multi-head block scores, one lane per block,
//                 fp32 fmaf chains in a fixed order (the order is what makes the
//                 selection reproducible bit for bit): score_tile for calls
//                 with many new tokens (a resident grid, each wave a range of
//                 consecutive tokens, the query as scalar operands); the decode
//                 form of score_kernel also appends and pools (at most one new
//                 token per sequence).
//   select        per-query top-k by (score desc, index asc): 4-pass 8-bit radix
//                 select in LDS, then an ascending compaction.
//   attn_decode   gated GQA softmax attention over the selected blocks + tail
//                 for decode-shaped calls (bf16, D = 128): 4-wave workgroups on
//                 splits of the selection list, QK and PV on bf16 MFMA, the
//                 top-k made in the kernel when it is given the scores.
//   attn_prefill_mfma  the same for prefill-sized calls: one wave per (token,
//                 KV head), QK and PV on bf16 MFMA (calls where some sequence has
//                 512 or more new tokens take the key-stationary path of
//                 qsa_prefill_ks.hip instead).
//   attn_split    the generic form (fp32, D = 64): one wave per (token, KV
//                 head, split); online softmax in base 2.
//   attn_combine  log-sum-exp merge of the splits and the sigmoid output gate.
//
// Semantics follow the QSA description of the Qwen4-Exp pages: MTPLX "Native
// Backend Components" (section "Qwen Sparse Attention"), the dev.to Qwen4-Exp
// article (section "Qwen Sparse Attention"), the LocalAI QSA-block commit on
// the llama.cpp PR #27739 page (indexer settings; gather, not mask), and
// "Porting Qwen4 to llama.cpp" (sections on selection semantics and on the
// direct indexed K/V endpoint).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "qsa_internal.h"

namespace qsa {
namespace {

#include "qsa_device.h"

// Debug builds only (QSA_COUNT_KEYS): every attention kernel adds the number
// of valid K/V rows it loads, per (token, KV head), to one device counter.
#ifdef QSA_COUNT_KEYS
__device__ unsigned long long g_keys_visited;
// Lane 0 of the calling wave adds the wave's count of set predicates.
#define QSA_COUNT_ROWS(pred)                                                              \
  do {                                                                                    \
    const unsigned long long n_ = __popcll(__ballot(pred));                               \
    if ((threadIdx.x & 63) == 0 && n_) atomicAdd(&g_keys_visited, n_);                    \
  } while (0)
#else
#define QSA_COUNT_ROWS(pred) \
  do {                       \
  } while (0)
#endif





// Element offset of row s of sequence b in the indexer-key cache, or -1.
__device__ __forceinline__ int64_t idx_row(const Geo& g, int b, int s) {
  if (s < 0 || s >= g.cap) return -1;
  if (g.page_table == nullptr) return ((int64_t)b * g.cap + s) * g.dI;
  const int page = g.page_table[(int64_t)b * g.max_pages + (s >> g.log2ps)];
  if (page < 0 || page >= g.n_pages) return -1;
  return ((int64_t)page * g.page_size + (s & (g.page_size - 1))) * g.dI;
}

// Monotone map of an fp32 score to uint32 (larger float -> larger key); -0 is
// folded onto +0 first so that equal scores give equal keys.
__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// 8-bit K/V storage ("Porting Qwen4 to llama.cpp", section "Quantized KV Is
// a Representation Contract").  OCP E4M3: 1 sign, 4 exponent bits (bias 7),
// 3 mantissa bits, exponent 0 subnormal (m * 2^-9), no infinities, 448 the
// largest finite value.  Encoding rounds to the nearest code, ties to the
// even code, and saturates at +-448; NaN encodes as 0x7F.  The mantissa LSB
// is the code's LSB, so rounding the scaled value to even is ties-to-even.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t sgn = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (!(a < 448.0f)) return (a != a) ? 0x7Fu : (sgn | 0x7Eu);
  if (a < 0.015625f) return sgn | (uint32_t)__builtin_rintf(a * 512.0f);  // m * 2^-9, m <= 8
  const int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;           // -6 .. 8
  const int m = (int)__builtin_rintf(__builtin_ldexpf(a, 3 - e));           // 8 .. 16
  return sgn | (uint32_t)((e + 7) * 8 + m - 8);  // m = 16 carries into the exponent
}


// One token's K and V rows (bf16 [Hkv][D], D = 128) into 8-bit caches, one
// wave: lane l holds elements 2l, 2l+1 of a row; rotated (Sylvester Hadamard,
// the standard butterfly order), scaled by 1/scale, encoded.  dst(kvh) is the
// element offset of the row in the cache (one byte per element).
template <typename RowOf>
__device__ __forceinline__ void store_rows_kv8(const Geo& g, const uint16_t* __restrict__ k_src,
                                               const uint16_t* __restrict__ v_src,
                                               uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                               RowOf dst) {
  const int lane = threadIdx.x & 63;
  for (int rw = 0; rw < 2 * g.Hkv; ++rw) {
    const int which = rw >= g.Hkv ? 1 : 0, kvh = rw - which * g.Hkv;
    const uint16_t* src = (which ? v_src : k_src) + (int64_t)kvh * 128;
    const uint32_t pr = *reinterpret_cast<const uint32_t*>(src + 2 * lane);
    float x0 = __uint_as_float(pr << 16), x1 = __uint_as_float(pr & 0xFFFF0000u);
    if (g.rot) {
      const float a = x0, b = x1;
      x0 = a + b;
      x1 = a - b;
#pragma unroll
      for (int dl = 1; dl < 64; dl <<= 1) {
        const bool up = (lane & dl) != 0;
        x0 = fwht_cross(x0, dl, up);
        x1 = fwht_cross(x1, dl, up);
      }
    }
    const float inv = which ? g.inv_v_scale : g.inv_k_scale;
    const uint32_t c = e4m3_encode(x0 * inv) | (e4m3_encode(x1 * inv) << 8);
    const int64_t d = dst(kvh);
    if (d >= 0) *reinterpret_cast<uint16_t*>((which ? vc : kc) + d + 2 * lane) = (uint16_t)c;
  }
}

// ---------------------------------------------------------------------------
// append + pool: grid (new token, role).  Role 0 (dispatched first) pools the
// block the token completes, if any; role 1 appends the token's rows.
template <typename E>
__global__ __launch_bounds__(256) void append_pool_kernel(
    Geo g, const E* __restrict__ k_new, const E* __restrict__ v_new,
    const E* __restrict__ kI_new, E* __restrict__ k_cache, E* __restrict__ v_cache,
    E* __restrict__ kI_cache, float* __restrict__ pooled, RopeTab rt) {
  const int t = blockIdx.x, tid = threadIdx.x;
  const bool pool_role = blockIdx.y == 0;
  if (pool_role && (pooled == nullptr || g.r == 0)) return;
  const QueryPos qp = query_pos(g, t);
  if (!qp.ok) return;
  constexpr int EPV = 16 / sizeof(E);  // elements per 16-byte copy
  if (!pool_role) {
    if (k_new != nullptr && g.kv8) {
      if constexpr (sizeof(E) == 2) {
        if (tid < 64)
          store_rows_kv8(g, reinterpret_cast<const uint16_t*>(k_new) + (int64_t)t * g.Hkv * 128,
                         reinterpret_cast<const uint16_t*>(v_new) + (int64_t)t * g.Hkv * 128,
                         reinterpret_cast<uint8_t*>(k_cache), reinterpret_cast<uint8_t*>(v_cache),
                         [&](int kvh) { return kv_row(g, qp.b, kvh, qp.p); });
      }
    } else if (k_new != nullptr) {
      const int units = g.D / EPV;
      const int per = g.Hkv * units;
      for (int u = tid; u < 2 * per; u += blockDim.x) {
        const int which = u / per, rem = u - which * per;
        const int kvh = rem / units, c = rem - kvh * units;
        const int64_t dst = kv_row(g, qp.b, kvh, qp.p);
        if (dst < 0) continue;
        const E* src = (which ? v_new : k_new) + ((int64_t)t * g.Hkv + kvh) * g.D + c * EPV;
        E* d = (which ? v_cache : k_cache) + dst + c * EPV;
        *reinterpret_cast<uint4*>(d) = *reinterpret_cast<const uint4*>(src);
      }
    }
    if (kI_new == nullptr) return;
    const int64_t dst = idx_row(g, qp.b, qp.p);
    if (dst >= 0) {
      for (int u = tid; u < g.dI / EPV; u += blockDim.x)
        *reinterpret_cast<uint4*>(kI_cache + dst + u * EPV) =
            *reinterpret_cast<const uint4*>(kI_new + (int64_t)t * g.dI + u * EPV);
    }
    return;
  }
  // The token that ends block j pools it.  Rows appended by this same call are
  // read from kI_new (another workgroup may not have stored them yet); older
  // rows come from the cache.  One thread per column adds the rows in token
  // order (the sequential fp32 sum); its loads go out kPoolBatch rows at a
  // time, all requested before the first add (rows in the cache first have
  // their addresses resolved, one thread per row).
  if (kI_new == nullptr || ((qp.p + 1) & (g.r - 1)) != 0) return;
  constexpr int kPoolBatch = 64;
  const int j = qp.p >> g.log2r;
  const int past = g.past_len[qp.b], t0 = g.cu_q[qp.b];
  const int dI = g.dI;
  __shared__ const E* rowp[kPoolBatch];  // a batch's row starts (cache rows' lookups)
  __shared__ int rowok[kPoolBatch];
  float acc = 0.0f;
  for (int s0 = j << g.log2r; s0 <= qp.p; s0 += kPoolBatch) {  // uniform
    const int n = qp.p + 1 - s0;  // rows left (the batch takes min(n, kPoolBatch))
    if (s0 >= past) {
      // all of the batch appended by this call: rows dI apart in kI_new
      if (tid < dI) {
        const E* src = kI_new + (int64_t)(t0 + s0 - past) * dI + tid;
        float v[kPoolBatch];
#pragma unroll
        for (int i = 0; i < kPoolBatch; ++i) v[i] = to_f32(src[(int64_t)min(i, n - 1) * dI]);
#pragma unroll
        for (int i = 0; i < kPoolBatch; ++i)
          if (i < n) acc = acc + v[i];
      }
    } else {
      // rows in the cache: one thread per row resolves its address (page
      // lookups all at once); absent rows read the token's own row, unused
      if (tid < kPoolBatch) {
        const int s = min(s0 + tid, qp.p);
        const E* ptr = kI_new + (int64_t)t * dI;
        int ok = tid < n;
        if (s >= past) {
          ptr = kI_new + (int64_t)(t0 + s - past) * dI;
        } else {
          const int64_t row = idx_row(g, qp.b, s);
          if (row >= 0) ptr = kI_cache + row;
          else ok = 0;
        }
        rowp[tid] = ptr;
        rowok[tid] = ok;
      }
      __syncthreads();
      if (tid < dI) {
        for (int c0 = 0; c0 < kPoolBatch && c0 < n; c0 += 16) {  // 16 loads in flight
          float v[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float x = to_f32(rowp[c0 + i][tid]);
            v[i] = rowok[c0 + i] ? x : 0.0f;
          }
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (c0 + i < n) acc = acc + v[i];
        }
      }
      __syncthreads();  // the next batch rewrites rowp
    }
  }
  float mean = acc * g.inv_r;
  if (g.idx_rope_dim > 0) {
    // Rotary indexer keys: the mean is rotated at the block's first position.
    __shared__ float mrow[128];
    if (tid < dI) mrow[tid] = mean;
    __syncthreads();
    if (tid < dI) mean = rope_at(mrow, tid, g.idx_rope_dim, rt.f, (int64_t)j << g.log2r);
  }
  if (tid < dI) pooled[((int64_t)qp.b * dI + tid) * g.pooled_ld + j] = mean;
}

// ---------------------------------------------------------------------------
// score: one wave per workgroup; grid (T, ceil(nbcap/64)) scoring workgroups,
// one lane per candidate block.  The pooled cache is column-major per
// sequence, so for each dimension x the wave reads 64 consecutive blocks (256
// contiguous bytes); each lane holds all d_I values of its block's pooled key
// in registers, loaded together.
// MODE 0: scoring only (the pooled cache is complete).
// MODE 1: the decode form, where every sequence has at most one new token,
// so no token of the call needs a row that another token appends.  Two more
// workgroups per token (grid y = 0, 1: dispatched first, so that their loads
// are not queued behind the scorers') do the rest of the step off the
// scorers' path: the first appends the token's K, V and
// indexer-key rows (read before the position is known); the second, when the
// token completes a block, pools that block (the new row from kI_new, the
// older rows from the cache, summed in token order as in append_pool_kernel),
// stores it in the pooled cache and writes its score (the scorers skip it).
// The scorers request a sequence's pooled keys only once its position shows
// that their group holds candidates: a batch's shorter sequences read no
// columns past their own blocks (requesting the keys before the position is
// known saves no time and reads up to the longest context for every token).

// Score of one pooled key held in LDS (pk[x], x < DI), computed by lane h < HI
// for head h, then summed over heads by lane 0 in head order: the same fmaf
// sequence as the scorers' (x ascending per head, then heads ascending).
template <int HIM, int DI>
__device__ __forceinline__ float score_one(const Geo& g, const float* qT, const float* wsh,
                                           const float* pk, float* hsum) {
  const int lane = threadIdx.x;
  if (lane < HIM) {
    float acc = 0.0f;
#pragma unroll
    for (int x = 0; x < DI; ++x) acc = fmaf(qT[x * HIM + lane], pk[x], acc);
    float a = g.idx_scale * acc;
    hsum[lane] = (a > 0.0f) ? a : 0.0f;
  }
  wave_sync();
  float s = 0.0f;
  for (int h = 0; h < HIM; ++h)
    if (h < g.HI) s = fmaf(wsh[h], hsum[h], s);
  return s;
}

template <typename E, int HIM, int DI, int MODE>
__global__ __launch_bounds__(64) void score_kernel(
    Geo g, const E* __restrict__ qI, const float* __restrict__ w, float* __restrict__ pooled,
    float* __restrict__ scores, const E* __restrict__ k_new, const E* __restrict__ v_new,
    const E* __restrict__ kI_new, E* __restrict__ k_cache, E* __restrict__ v_cache,
    E* __restrict__ kI_cache, RopeTab rt) {
  constexpr bool APPEND = MODE != 0;
  constexpr int EPV = 16 / sizeof(E);  // elements per 16-byte copy
  __shared__ __attribute__((aligned(16))) float qT[DI * HIM];  // [x][h]
  __shared__ float wsh[HIM];
  const int t = blockIdx.x, lane = threadIdx.x;
  // decode form: y = 0 appends, y = 1 pools, y >= 2 scores group y - 2
  const int role = APPEND ? (int)blockIdx.y : -1;
  const int group = APPEND ? (int)blockIdx.y - 2 : (int)blockIdx.y;

  if (APPEND && role == 0) {
    // This token's new rows, 16 bytes per lane and load (the first 4 per
    // lane held across the position and page lookups).
    const int kv_units = 2 * g.Hkv * (g.D / EPV), per = kv_units >> 1, units = g.D / EPV;
    uint4 kvv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = min(lane + 64 * i, kv_units - 1);
      const int which = u >= per ? 1 : 0;
      kvv[i] = *reinterpret_cast<const uint4*>((which ? v_new : k_new) +
                                               (int64_t)t * g.Hkv * g.D + (u - which * per) * EPV);
    }
    const uint4 kiv =
        *reinterpret_cast<const uint4*>(kI_new + (int64_t)t * DI + min(lane, DI / EPV - 1) * EPV);
    const QueryPos qp = query_pos(g, t);
    if (!qp.ok) return;
    if (g.kv8) {  // 8-bit storage: rotated, scaled and encoded rows
      if constexpr (sizeof(E) == 2)
        store_rows_kv8(g, reinterpret_cast<const uint16_t*>(k_new) + (int64_t)t * g.Hkv * 128,
                       reinterpret_cast<const uint16_t*>(v_new) + (int64_t)t * g.Hkv * 128,
                       reinterpret_cast<uint8_t*>(k_cache), reinterpret_cast<uint8_t*>(v_cache),
                       [&](int kvh) { return kv_row(g, qp.b, kvh, qp.p); });
    }
    for (int u = lane; u < (g.kv8 ? 0 : kv_units); u += 64) {
      const int which = u >= per ? 1 : 0, rem = u - which * per;
      const int kvh = rem / units, c = rem - kvh * units;
      const int64_t dst = kv_row(g, qp.b, kvh, qp.p);
      if (dst < 0) continue;
      const int i = (u - lane) >> 6;
      uint4 v;
      if (i < 4) {
        v = kvv[0];
#pragma unroll
        for (int ii = 1; ii < 4; ++ii) v = (i == ii) ? kvv[ii] : v;
      } else {
        v = *reinterpret_cast<const uint4*>((which ? v_new : k_new) +
                                            ((int64_t)t * g.Hkv + kvh) * g.D + c * EPV);
      }
      *reinterpret_cast<uint4*>((which ? v_cache : k_cache) + dst + c * EPV) = v;
    }
    const int64_t drow = idx_row(g, qp.b, qp.p);
    if (drow >= 0 && lane < DI / EPV) *reinterpret_cast<uint4*>(kI_cache + drow + lane * EPV) = kiv;
    return;
  }

  // The query and the head weights do not depend on the token's position:
  // staged before the sequence search so the loads overlap.
  {
    const int HI = g.HI;
    for (int e = lane; e < DI * HIM; e += 64) {
      const int x = e / HIM, h = e - x * HIM;
      qT[e] = h < HI ? to_f32(qI[((int64_t)t * HI + h) * DI + x]) : 0.0f;
    }
    if (lane < HIM) wsh[lane] = lane < HI ? w[(int64_t)t * HI + lane] : 0.0f;
  }

  if (APPEND && role == 1) {
    const QueryPos qp = query_pos(g, t);
    if (!qp.ok || ((qp.p + 1) & (g.r - 1)) != 0) return;
    // Rows of the block first (one page lookup per row, all lanes at once;
    // -2 marks the new row, -1 a row outside the cache), then 64 rows at a
    // time: every lane loads its column(s) of all 64 rows (all loads in
    // flight, at addresses chosen by selects), then adds them in token order.
    constexpr int CPT = DI >= 64 ? DI / 64 : 1;  // columns per lane
    __shared__ __attribute__((aligned(16))) int32_t prow[256];  // block_size <= 256
    __shared__ float newpool[DI];
    __shared__ float hsum[HIM];
    const int nb = (qp.p + 1) >> g.log2r, jnew = nb - 1;
    const int s0 = jnew << g.log2r;
    for (int rr = lane; rr < g.r; rr += 64) {
      const int sr = s0 + rr;
      const int64_t row = sr == qp.p ? -2 : idx_row(g, qp.b, sr);
      prow[rr] = row >= 0 ? (int32_t)(row / DI) : (int32_t)row;
    }
    wave_sync();
    const E* newrow = kI_new + (int64_t)t * DI;
    float acc[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[c] = 0.0f;
    for (int c0 = 0; c0 < g.r; c0 += 64) {
      const int nrow = min(64, g.r - c0);
      float v[CPT][64];
#pragma unroll
      for (int i4 = 0; i4 < 16; ++i4) {
        const int4 pr4 = *reinterpret_cast<const int4*>(&prow[min(c0 + 4 * i4, 252)]);
        const int32_t prs[4] = {pr4.x, pr4.y, pr4.z, pr4.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // (rows past the block read row 0 of the cache and count as zero)
          const int32_t pr = c0 + 4 * i4 + k < g.r ? prs[k] : -1;
          const E* src = pr == -2 ? newrow : kI_cache + (int64_t)max(pr, 0) * DI;
#pragma unroll
          for (int c = 0; c < CPT; ++c) {
            const int x = min(lane + 64 * c, DI - 1);
            const float f = to_f32(src[x]);
            v[c][4 * i4 + k] = pr == -1 ? 0.0f : f;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 64; ++i)
#pragma unroll
        for (int c = 0; c < CPT; ++c)
          if (i < nrow) acc[c] = acc[c] + v[c][i];
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int x = lane + 64 * c;
      if (x < DI) newpool[x] = acc[c] * g.inv_r;
    }
    wave_sync();
    if (g.idx_rope_dim > 0) {
      // Rotary indexer keys: the mean is rotated at the block's first position.
      float rv[CPT];
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int x = min(lane + 64 * c, DI - 1);
        rv[c] = rope_at(newpool, x, g.idx_rope_dim, rt.f, (int64_t)s0);
      }
      wave_sync();
#pragma unroll
      for (int c = 0; c < CPT; ++c)
        if (lane + 64 * c < DI) newpool[lane + 64 * c] = rv[c];
      wave_sync();
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int x = lane + 64 * c;
      if (x < DI) pooled[((int64_t)qp.b * DI + x) * g.pooled_ld + jnew] = newpool[x];
    }
    const float sc = score_one<HIM, DI>(g, qT, wsh, newpool, hsum);
    if (lane == 0 && jnew < g.nbcap) scores[(int64_t)t * g.nbcap + jnew] = sc;
    return;
  }

  // Scorer.  (Buffer loads: one column offset per lane, the row offset in a
  // scalar; unconditional, at a clamped column.)
  const int j = group * 64 + lane;
  float pk[DI];
  auto load_keys = [&](int b) {
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(pooled + (int64_t)b * DI * g.pooled_ld, (uint32_t)(DI * g.pooled_ld * 4));
    const uint32_t col = (uint32_t)min(j, g.pooled_ld - 1) * 4u;
#pragma unroll
    for (int x = 0; x < DI; ++x)
      pk[x] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                            rs, col, (uint32_t)(x * g.pooled_ld * 4), 0));
  };
  const QueryPos qp = query_pos(g, t);
  const int nb = qp.ok ? ((qp.p + 1) >> g.log2r) : 0;
  if (group * 64 < nb) load_keys(qp.b);
  // (decode form) the block this token completes is scored by the pooler
  const int jnew = (APPEND && qp.ok && ((qp.p + 1) & (g.r - 1)) == 0) ? nb - 1 : -1;
  __syncthreads();
  float s = 0.0f;
  if (group * 64 < nb) {
    float acc[HIM];
#pragma unroll
    for (int h = 0; h < HIM; ++h) acc[h] = 0.0f;
    // Chunks of XC dimensions in a loop that is not unrolled (so the query
    // reads of one chunk are not hoisted into registers ahead of the others),
    // the chunk's keys picked out of the registers by selects; each head's
    // chain advances x in ascending order.
    constexpr int XC = DI <= 32 ? 16 : 32;
    constexpr int NCH = DI / XC;
#pragma unroll 1
    for (int c = 0; c < NCH; ++c) {
      float pc[XC];
#pragma unroll
      for (int xx = 0; xx < XC; ++xx) {
        float v = pk[xx];
#pragma unroll
        for (int cc = 1; cc < NCH; ++cc) v = (c == cc) ? pk[cc * XC + xx] : v;
        pc[xx] = v;
      }
#pragma unroll
      for (int xx = 0; xx < XC; ++xx) {
        const float4* qrow = reinterpret_cast<const float4*>(qT + (c * XC + xx) * HIM);
#pragma unroll
        for (int h4 = 0; h4 < HIM / 4; ++h4) {
          const float4 qv = qrow[h4];
          acc[4 * h4 + 0] = fmaf(qv.x, pc[xx], acc[4 * h4 + 0]);
          acc[4 * h4 + 1] = fmaf(qv.y, pc[xx], acc[4 * h4 + 1]);
          acc[4 * h4 + 2] = fmaf(qv.z, pc[xx], acc[4 * h4 + 2]);
          acc[4 * h4 + 3] = fmaf(qv.w, pc[xx], acc[4 * h4 + 3]);
        }
      }
    }
    const int HI = g.HI;
#pragma unroll
    for (int h = 0; h < HIM; ++h) {
      if (h < HI) {
        float a = g.idx_scale * acc[h];
        a = (a > 0.0f) ? a : 0.0f;
        s = fmaf(wsh[h], a, s);
      }
    }
  }
  if (j < g.nbcap && j != jnew) scores[(int64_t)t * g.nbcap + j] = (j < nb) ? s : -INFINITY;
}

// score, the form for calls that bring many tokens at once (prefill chunks,
// ragged prefill, verify).  The work is T x ceil(nbcap / 64) units (token,
// group of 64 candidate blocks), group-major; a grid of as many 4-wave
// workgroups as the GPU holds at once gives every wave an equal contiguous
// range of units (the counts differ by at most one), so no wave waits for a
// second round and a wave's tokens are consecutive within a group.  Lanes
// are the group's blocks; a sequence's pooled keys are loaded into registers
// once for all of its tokens in the range.  A token's query and head weights
// are the same for every lane, so they are read with scalar loads and enter
// each fmaf as its scalar operand (broadcasting them through LDS would move
// 256 bytes per value and wave, more than the LDS delivers for one fmaf per
// lane and value).  Every score is the same fmaf chain as the per-token form
// (x ascending per head, then heads ascending).
template <typename E, int HIM, int DI>
__global__ __launch_bounds__(256) void score_tile_kernel(Geo g, const E* __restrict__ qI,
                                                         const float* __restrict__ w,
                                                         const float* __restrict__ pooled,
                                                         float* __restrict__ scores) {
  __shared__ int tinfo[4][64][2];  // (sequence, complete blocks) of up to 64 tokens
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t T = g.T, groups = (g.nbcap + 63) / 64, U = T * groups;
  const int64_t nw = (int64_t)gridDim.x * 4, gw = (int64_t)blockIdx.x * 4 + wv;
  const int64_t u_end = (gw + 1) * U / nw;
  const int HI = g.HI;
  float pk[DI];
  int kb = -1, kg = -1;  // sequence and group whose keys pk holds
  for (int64_t u = gw * U / nw; u < u_end;) {
    const int group = (int)(u / T), t0 = (int)(u - (int64_t)group * T);
    const int nt = (int)min<int64_t>(min<int64_t>(u_end - u, T - t0), 64);
    const int j = group * 64 + lane;
    // Positions of the next nt tokens, one lane per token: the first one's
    // sequence by search (the whole wave), then each lane steps over the
    // sequence boundaries up to its token.
    const QueryPos q0 = query_pos(g, t0);
    wave_sync();  // (the previous tokens' entries have been read)
    if (lane < nt) {
      const int t = t0 + lane;
      int b = g.one_q ? t : q0.b;
      if (!g.one_q)
        while (b + 1 < g.B && g.cu_q[b + 1] <= t) ++b;
      const int p = g.one_q ? g.past_len[t] : g.past_len[b] + (t - g.cu_q[b]);
      const bool ok = p >= 0 && p < g.cap;
      tinfo[wv][lane][0] = b;
      tinfo[wv][lane][1] = ok ? ((p + 1) >> g.log2r) : 0;
    }
    wave_sync();
    for (int i = 0; i < nt; ++i) {
      const int t = t0 + i;
      const int b = __builtin_amdgcn_readfirstlane(tinfo[wv][i][0]);
      const int nb = __builtin_amdgcn_readfirstlane(tinfo[wv][i][1]);
      float s = 0.0f;
      if (group * 64 < nb) {
        if (b != kb || group != kg) {
          const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(pooled + (int64_t)b * DI * g.pooled_ld,
                                                        (uint32_t)(DI * g.pooled_ld * 4));
          const uint32_t col = (uint32_t)min(j, g.pooled_ld - 1) * 4u;
#pragma unroll
          for (int x = 0; x < DI; ++x)
            pk[x] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                  rs, col, (uint32_t)(x * g.pooled_ld * 4), 0));
          kb = b;
          kg = group;
          // All key loads complete here, so the chains below carry no
          // per-use waits for loads that only this branch issues.
          __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        }
        // The query words of HB heads are requested together (at most 32
        // scalar registers) and waited for once; the head weights first.
        constexpr int DW = DI * (int)sizeof(E) / 4;  // 32-bit words per head row
        constexpr int HB = DW >= 32 ? 1 : (32 / DW < HIM ? 32 / DW : HIM);
        float wh[HIM];
#pragma unroll
        for (int h = 0; h < HIM; ++h) wh[h] = w[(int64_t)t * HI + min(h, HI - 1)];
        const uint32_t* qt = reinterpret_cast<const uint32_t*>(qI) + (int64_t)t * HI * DW;
#pragma unroll
        for (int h0 = 0; h0 < HIM; h0 += HB) {
          if (h0 < HI) {
            uint32_t qw[HB][DW];
#pragma unroll
            for (int hh = 0; hh < HB; ++hh)
#pragma unroll
              for (int wd = 0; wd < DW; ++wd) qw[hh][wd] = qt[min(h0 + hh, HI - 1) * DW + wd];
#pragma unroll
            for (int hh = 0; hh < HB; ++hh) {
              if (h0 + hh < HI) {
                float acc = 0.0f;
#pragma unroll
                for (int wd = 0; wd < DW; ++wd) {
                  const uint32_t qd = qw[hh][wd];
                  if constexpr (sizeof(E) == 2) {
                    // bf16 pairs: the low half is the even dimension
                    acc = fmaf(__builtin_bit_cast(float, qd << 16), pk[2 * wd], acc);
                    acc = fmaf(__builtin_bit_cast(float, qd & 0xffff0000u), pk[2 * wd + 1], acc);
                  } else {
                    acc = fmaf(__builtin_bit_cast(float, qd), pk[wd], acc);
                  }
                }
                float a = g.idx_scale * acc;
                a = (a > 0.0f) ? a : 0.0f;
                s = fmaf(wh[h0 + hh], a, s);
              }
            }
          }
        }
      }
      if (j < g.nbcap) scores[(int64_t)t * g.nbcap + j] = (j < nb) ? s : -INFINITY;
    }
    u += nt;
  }
}

// ---------------------------------------------------------------------------
// Inclusive prefix sum over one wave on DPP: shifts by 1, 2, 4, 8 lanes inside
// each 16-lane row (zero shifted in), then the row totals are carried by the
// lane-15 and lane-31 broadcasts.  No LDS round trips.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Exclusive prefix sum over one wave.
__device__ __forceinline__ int wave_excl_scan(int v) { return wave_incl_scan(v) - v; }

// Exclusive prefix sum over a 256-thread workgroup (sh: 4 ints of LDS).
__device__ __forceinline__ int block_excl_scan(int v, int* total, int* sh) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) sh[wid] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = sh[i];
    off += (i < wid) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + x - v;
}

// Top-k over keys held 8 per thread by a 256-thread workgroup: thread tid owns
// the candidates [jb, jb + jn), jn <= 8, in index order (thread order = index
// order, so the kept ids come out ascending).  The ids of the k largest keys,
// ties to the lowest id, go to out (LDS or global).
// 8-bit radix passes over the keys in registers (LDS histograms).
__device__ __forceinline__ void block_radix_topk(const uint32_t (&kr)[8], int jb, int jn, int k,
                                                 int32_t* out) {
  // Two histograms: while wave 0 scans one, the other is cleared for the next
  // pass, so a pass costs two barriers.  The passes stop early once the keys
  // that share the digits found so far are exactly the ones still wanted:
  // then all of them are kept, whatever their lower bits.
  __shared__ __attribute__((aligned(16))) uint32_t hist[2][256];
  __shared__ uint32_t s_prefix;
  __shared__ int s_want, s_cnt;
  __shared__ int sh[4];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint32_t prefix = 0, mask = 0;
  int want = k;
  hist[0][tid] = 0;
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    uint32_t* hc = hist[pass & 1];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e < jn && (kr[e] & mask) == prefix) atomicAdd(&hc[(kr[e] >> shift) & 255u], 1u);
    __syncthreads();
    if (wid == 0) {
      // lane owns digits 255-4*lane .. 252-4*lane (descending)
      const uint4 h4 = *reinterpret_cast<const uint4*>(&hc[252 - 4 * lane]);
      const int c[4] = {(int)h4.w, (int)h4.z, (int)h4.y, (int)h4.x};
      int above = wave_excl_scan(c[0] + c[1] + c[2] + c[3]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (above < want && above + c[i] >= want) {
          s_prefix = prefix | ((uint32_t)(255 - 4 * lane - i) << shift);
          s_want = want - above;
          s_cnt = c[i];
        }
        above += c[i];
      }
    }
    if (pass < 3) hist[(pass + 1) & 1][tid] = 0;
    __syncthreads();
    prefix = s_prefix;
    want = s_want;
    mask |= 255u << shift;
    if (s_cnt == want) break;  // (the same value in every thread)
  }
  // Keep keys above the found digits, and the first `want` keys that share
  // them in index order: one packed scan gives each thread both counts.
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (e < jn) {
      const uint32_t km = kr[e] & mask;
      n_gt += km > prefix ? 1 : 0;
      n_eq += km == prefix ? 1 : 0;
    }
  }
  int tot;
  const int before = block_excl_scan((n_gt << 16) | n_eq, &tot, sh);
  int pos = (before >> 16) + min(before & 0xffff, want);
  int eqr = before & 0xffff;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (e < jn) {
      const uint32_t km = kr[e] & mask;
      const bool eq = km == prefix;
      if (km > prefix || (eq && eqr < want)) {
        if (pos < k) out[pos] = jb + e;
        ++pos;
      }
      eqr += eq ? 1 : 0;
    }
  }
}

// select: one 256-thread workgroup per query.  Thread tid owns the contiguous
// candidates [tid*per, tid*per + per); with per <= 8 (nb <= 2048) their keys
// stay in registers across the passes.
//   4 passes of an 8-bit radix select find the k-th largest key K and how
//   many keys equal to K are kept (the lowest-index ones: ties go to the
//   lowest block index); a final pass writes the kept ids in ascending order.
template <bool CACHED>
__device__ __forceinline__ void select_impl(const Geo& g, const float* __restrict__ srow, int nb,
                                            int32_t* __restrict__ out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix;
  __shared__ int s_want;
  __shared__ int sh[4];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, k = g.k;
  const int per = (nb + 255) >> 8;
  const int jb = tid * per;
  const int jn = max(0, min(per, nb - jb));  // candidates this thread owns
  uint32_t kr[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  uint32_t prefix = 0, mask = 0;
  int want = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    if (CACHED) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e < jn && (kr[e] & mask) == prefix) atomicAdd(&hist[(kr[e] >> shift) & 255u], 1u);
    } else {
      for (int e = 0; e < jn; ++e) {
        const uint32_t key = score_key(srow[jb + e]);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    if (wid == 0) {
      // lane owns digits 255-4*lane .. 252-4*lane (descending)
      int c[4], tot = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = (int)hist[255 - 4 * lane - i];
        tot += c[i];
      }
      int above = wave_excl_scan(tot);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (above < want && above + c[i] >= want) {
          s_prefix = prefix | ((uint32_t)(255 - 4 * lane - i) << shift);
          s_want = want - above;
        }
        above += c[i];
      }
    }
    __syncthreads();
    prefix = s_prefix;
    want = s_want;
    mask |= 255u << shift;
  }
  // Keep keys > prefix, and the first `want` keys == prefix in index order.
  // Pass 1 counts equal keys (for their global rank) and kept keys; pass 2
  // writes the kept ids at their ascending positions.
  int n_eq = 0;
  if (CACHED) {
#pragma unroll
    for (int e = 0; e < 8; ++e) n_eq += (e < jn && kr[e] == prefix) ? 1 : 0;
  } else {
    for (int e = 0; e < jn; ++e) n_eq += (score_key(srow[jb + e]) == prefix) ? 1 : 0;
  }
  int tot;
  const int eq_before = block_excl_scan(n_eq, &tot, sh);
  int n_take = 0;
  {
    int eqr = eq_before;
    if (CACHED) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (e < jn) {
          const bool eq = kr[e] == prefix;
          n_take += (kr[e] > prefix || (eq && eqr < want)) ? 1 : 0;
          eqr += eq ? 1 : 0;
        }
      }
    } else {
      for (int e = 0; e < jn; ++e) {
        const uint32_t key = score_key(srow[jb + e]);
        const bool eq = key == prefix;
        n_take += (key > prefix || (eq && eqr < want)) ? 1 : 0;
        eqr += eq ? 1 : 0;
      }
    }
  }
  int pos = block_excl_scan(n_take, &tot, sh);
  {
    int eqr = eq_before;
    if (CACHED) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (e < jn) {
          const bool eq = kr[e] == prefix;
          if (kr[e] > prefix || (eq && eqr < want)) {
            if (pos < k) out[pos] = jb + e;
            ++pos;
          }
          eqr += eq ? 1 : 0;
        }
      }
    } else {
      for (int e = 0; e < jn; ++e) {
        const uint32_t key = score_key(srow[jb + e]);
        const bool eq = key == prefix;
        if (key > prefix || (eq && eqr < want)) {
          if (pos < k) out[pos] = jb + e;
          ++pos;
        }
        eqr += eq ? 1 : 0;
      }
    }
  }
  (void)lane;
}

// select, up to 2048 candidate blocks: one 256-thread workgroup per query,
// 8 keys per thread (block_radix_topk).  The scores are read before the query's
// position is known (the row is -inf past its candidates), so that both
// loads overlap.
constexpr int kSelectMaxBlocks = 2048;
__global__ __launch_bounds__(256) void select_kernel(Geo g, const float* __restrict__ scores,
                                                     int32_t* __restrict__ sel,
                                                     int32_t* __restrict__ n_blocks) {
  const int t = blockIdx.x, tid = threadIdx.x, k = g.k;
  const float* srow = scores + (int64_t)t * g.nbcap;
  const int per = (g.nbcap + 255) >> 8;
  const int jb = tid * per;
  // Unconditional loads (clamped index, value masked after): conditional
  // loads would each wait for the previous one.
  uint32_t kr[8];
  const int jlast = max(g.nbcap - 1, 0);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float v = srow[min(jb + e, jlast)];
    kr[e] = (e < per && jb + e < g.nbcap) ? score_key(v) : 0u;
  }
  const QueryPos qp = query_pos(g, t);
  const int nb = qp.ok ? min((qp.p + 1) >> g.log2r, g.nbcap) : 0;
  int32_t* out = sel + (int64_t)t * k;
  if (nb <= k) {  // every candidate is kept
    for (int i = tid; i < k; i += 256) out[i] = i < nb ? i : -1;
  } else {
    block_radix_topk(kr, jb, max(0, min(per, nb - jb)), k, out);
  }
  if (tid == 0) n_blocks[t] = min(k, nb);
}

// select, up to 512 candidate blocks: one wave per query, four queries per
// workgroup, lane l owning candidates [8 l, 8 l + 8).  The same 8-bit radix
// passes and the same tie rule as block_radix_topk, on a histogram of the
// wave's own in LDS: no workgroup barrier anywhere, so the calls with many
// queries (prefill) keep four times as many selections in flight per CU as
// with a workgroup per query.  The LDS performs one wave's operations in the
// order the wave issues them, so nothing has to wait between clearing the
// histogram, counting into it and reading it back; the wavefront-scope fence
// and wave barrier only keep the compiler from reordering those phases.
constexpr int kSelectWaveBlocks = 512;
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}
__global__ __launch_bounds__(256) void select_wave_kernel(Geo g, const float* __restrict__ scores,
                                                          int32_t* __restrict__ sel,
                                                          int32_t* __restrict__ n_blocks) {
  __shared__ __attribute__((aligned(16))) uint32_t hist_all[4][256];
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63, k = g.k;
  const int t = blockIdx.x * 4 + wid;
  if (t >= g.T) return;  // (whole waves; no workgroup barrier follows)
  uint32_t* hc = hist_all[wid];
  const float* srow = scores + (int64_t)t * g.nbcap;
  const int jb = 8 * lane;
  // Unconditional loads at clamped indices, masked after with an AND (a
  // select would let the compiler move each load under its own branch and
  // wait for it there).
  uint32_t kr[8];
  const int jlast = max(g.nbcap - 1, 0);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float v = srow[min(jb + e, jlast)];
    kr[e] = score_key(v) & (0u - (uint32_t)(jb + e < g.nbcap));
  }
  const QueryPos qp = query_pos(g, t);
  const int nb = qp.ok ? min((qp.p + 1) >> g.log2r, g.nbcap) : 0;
  int32_t* out = sel + (int64_t)t * k;
  if (lane == 0) n_blocks[t] = min(k, nb);
  if (nb <= k) {  // every candidate is kept
    for (int i = lane; i < k; i += 64) out[i] = i < nb ? i : -1;
    return;
  }
  const int jn = max(0, min(8, nb - jb));
  uint32_t prefix = 0, mask = 0;
  int want = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    *reinterpret_cast<uint4*>(&hc[4 * lane]) = make_uint4(0u, 0u, 0u, 0u);
    wave_lds_sync();
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e < jn && (kr[e] & mask) == prefix) atomicAdd(&hc[(kr[e] >> shift) & 255u], 1u);
    wave_lds_sync();
    // lane owns digits 255-4*lane .. 252-4*lane (descending)
    const uint4 h4 = *reinterpret_cast<const uint4*>(&hc[252 - 4 * lane]);
    wave_lds_sync();
    const int c[4] = {(int)h4.w, (int)h4.z, (int)h4.y, (int)h4.x};
    int above = wave_excl_scan(c[0] + c[1] + c[2] + c[3]);
    int hit = 0, n_want = 0, n_cnt = 0;
    uint32_t n_prefix = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (above < want && above + c[i] >= want) {
        hit = 1;
        n_prefix = prefix | ((uint32_t)(255 - 4 * lane - i) << shift);
        n_want = want - above;
        n_cnt = c[i];
      }
      above += c[i];
    }
    // exactly one lane holds the digit (nb > k keys were counted in pass 0,
    // and every later pass counts the want-th key's digit group)
    const int src = __builtin_ctzll(__ballot(hit));
    prefix = (uint32_t)__builtin_amdgcn_readlane((int)n_prefix, src);
    want = __builtin_amdgcn_readlane(n_want, src);
    const int cnt = __builtin_amdgcn_readlane(n_cnt, src);
    mask |= 255u << shift;
    if (cnt == want) break;
  }
  // Keys above the found digits, and the first `want` keys that share them in
  // index order: one packed scan gives each lane both counts.
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (e < jn) {
      const uint32_t km = kr[e] & mask;
      n_gt += km > prefix ? 1 : 0;
      n_eq += km == prefix ? 1 : 0;
    }
  }
  const int before = wave_excl_scan((n_gt << 16) | n_eq);
  int pos = (before >> 16) + min(before & 0xffff, want);
  int eqr = before & 0xffff;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (e < jn) {
      const uint32_t km = kr[e] & mask;
      const bool eq = km == prefix;
      if (km > prefix || (eq && eqr < want)) {
        if (pos < k) out[pos] = jb + e;
        ++pos;
      }
      eqr += eq ? 1 : 0;
    }
  }
}

// select, more candidate blocks: one 256-thread workgroup per query, 8-bit
// radix passes over the scores in memory.
__global__ __launch_bounds__(256) void select_large_kernel(Geo g, const float* __restrict__ scores,
                                                           int32_t* __restrict__ sel,
                                                           int32_t* __restrict__ n_blocks) {
  const int t = blockIdx.x, tid = threadIdx.x, k = g.k;
  const QueryPos qp = query_pos(g, t);
  // (min with the score row length only matters for inconsistent metadata)
  const int nb = qp.ok ? min((qp.p + 1) >> g.log2r, g.nbcap) : 0;
  int32_t* out = sel + (int64_t)t * k;
  if (nb <= k) {  // every candidate is kept
    for (int i = tid; i < k; i += 256) out[i] = i < nb ? i : -1;
    if (tid == 0) n_blocks[t] = nb;
    return;
  }
  select_impl<false>(g, scores + (int64_t)t * g.nbcap, nb, out);
  if (tid == 0) n_blocks[t] = k;
}

// ---------------------------------------------------------------------------
// Attention.
template <typename E> struct QStage;
template <> struct QStage<uint16_t> { typedef uint32_t T; static constexpr int per = 2; };
template <> struct QStage<float> { typedef float T; static constexpr int per = 1; };

struct ListInfo {
  int n_list;   // tokens in the selection list (blocks then tail)
  int nsel_tok; // tokens coming from selected blocks (nblocks * r)
  int nb;       // complete candidate blocks
  int tail0;    // first tail token (r * nb)
};

__device__ __forceinline__ ListInfo list_info(const Geo& g, const QueryPos& qp,
                                              const int32_t* nblk, int t) {
  ListInfo L = {0, 0, 0, 0};
  if (!qp.ok) return L;
  const int n = qp.p + 1;
  if (g.r == 0) {
    L.n_list = n;
    return L;
  }
  L.nb = n >> g.log2r;
  int nk = nblk[t];
  nk = max(0, min(nk, min(g.k, L.nb)));
  L.nsel_tok = nk << g.log2r;
  L.tail0 = L.nb << g.log2r;
  L.n_list = L.nsel_tok + (n - L.tail0);
  return L;
}

// Physical token of list position i (blocks ascending, then the tail); -1 if
// the selection entry is not a valid candidate block.
__device__ __forceinline__ int list_token(const Geo& g, const ListInfo& L,
                                          const int32_t* srow, int i) {
  if (g.r == 0) return i;
  if (i < L.nsel_tok) {
    const int blk = srow[i >> g.log2r];
    return (blk >= 0 && blk < L.nb) ? (blk << g.log2r) + (i & (g.r - 1)) : -1;
  }
  return L.tail0 + (i - L.nsel_tok);
}


// A split covers the 64-token tiles [tiles * s / S, tiles * (s + 1) / S) of the
// longest list (S = n_splits): the same boundaries for every unit, so splits
// differ by at most one tile.
__device__ __forceinline__ int split_begin(const AttnPlan& plan, int split) {
  return 64 * (int)(((int64_t)split * plan.tiles) / plan.n_splits);
}

// Split merge: one workgroup per (token, KV head) unit, launched after the
// attention kernel (the kernel boundary makes every split's partial visible).
// Partials: [split][G][D] o, then [G] m, then [G] l (base-2 log-sum-exp
// state); a unit whose query lies outside the capacities has l = -1 in every
// split and is skipped.  The gate and the partials of kCombineBatch splits are
// loaded together and merged under a running maximum: one memory round trip
// per batch of splits.
constexpr int kCombineBatch = 16;
template <typename E, int G, int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(Geo g, AttnPlan plan,
                                                           const float* __restrict__ part,
                                                           const E* __restrict__ gate,
                                                           E* __restrict__ out) {
  constexpr int NT = 256;
  constexpr int SP = G * (D + 2);
  constexpr int EPT = (G * D >= NT) ? G * D / NT : 1;  // elements per thread, inside one head
  static_assert(D % EPT == 0, "combine layout");
  const int unit = blockIdx.x;
  const int t = unit / g.Hkv, kvh = unit - t * g.Hkv;
  const int e0 = threadIdx.x * EPT;
  if (e0 >= G * D) return;
  const int h = e0 / D, d0 = e0 - h * D;
  const int64_t ob = ((int64_t)t * g.Hq + kvh * G + h) * D + d0;
  float gt[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) gt[i] = to_f32(gate[ob + i]);
  const int S = plan.n_splits;
  const float* P0 = part + (int64_t)unit * S * SP;
  const float flag = P0[G * D + G];
  float M = -INFINITY, Ls = 0.0f, O[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) O[i] = 0.0f;
  for (int s0 = 0; s0 < S; s0 += kCombineBatch) {
    float mv[kCombineBatch], lv[kCombineBatch], ov[kCombineBatch][EPT];
#pragma unroll
    for (int c = 0; c < kCombineBatch; ++c) {
      const float* ps = P0 + (int64_t)min(s0 + c, S - 1) * SP;
      mv[c] = ps[G * D + h];
      lv[c] = ps[G * D + G + h];
#pragma unroll
      for (int i = 0; i < EPT; ++i) ov[c][i] = ps[h * D + d0 + i];
    }
    float cm = M;
#pragma unroll
    for (int c = 0; c < kCombineBatch; ++c)
      if (s0 + c < S) cm = fmaxf(cm, mv[c]);
    const float a = (M == -INFINITY) ? 0.0f : exp2f(M - cm);
    Ls *= a;
#pragma unroll
    for (int i = 0; i < EPT; ++i) O[i] *= a;
#pragma unroll
    for (int c = 0; c < kCombineBatch; ++c) {
      const float w = (s0 + c < S && mv[c] != -INFINITY) ? exp2f(mv[c] - cm) : 0.0f;
      Ls = fmaf(lv[c], w, Ls);
#pragma unroll
      for (int i = 0; i < EPT; ++i) O[i] = fmaf(ov[c][i], w, O[i]);
    }
    M = cm;
  }
  if (flag < 0.0f) return;
  const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
#pragma unroll
  for (int i = 0; i < EPT; ++i) O[i] *= inv;
  if constexpr (D == 128) {
    if (g.kv8) kv8_output(g, O, d0 / EPT);
  }
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const float sg = 1.0f / (1.0f + expf(-gt[i]));
    out[ob + i] = from_f32<E>(O[i] * sg);
  }
}

constexpr int kWaves = 4;       // waves per workgroup of the bf16 D=128 kernel

template <typename E, int G, int D>
__global__ __launch_bounds__(64) void attn_split_kernel(
    Geo g, AttnPlan plan, const E* __restrict__ q, const E* __restrict__ kc,
    const E* __restrict__ vc, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ nblk, const E* __restrict__ gate, E* __restrict__ out,
    float* __restrict__ part) {
  typedef typename QStage<E>::T QT;
  constexpr int QW = D / QStage<E>::per;  // staged q words per head
  constexpr int DPL = D / 64;             // output dims per lane
  __shared__ QT qs[G * QW];
  __shared__ float ps[64 * G];
  __shared__ int64_t rows[64];

  const int unit = blockIdx.x, split = blockIdx.y, lane = threadIdx.x;
  const int t = unit / g.Hkv, kvh = unit - t * g.Hkv;
  const QueryPos qp = query_pos(g, t);
  const ListInfo L = list_info(g, qp, nblk, t);
  const int i0 = split_begin(plan, split);
  const int i1 = min(split_begin(plan, split + 1), L.n_list);
  const int h0 = kvh * G;

  float m[G], l[G], o[G][DPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int d = 0; d < DPL; ++d) o[h][d] = 0.0f;
  }

  if (i0 < i1) {
    const QT* qsrc = reinterpret_cast<const QT*>(q + ((int64_t)t * g.Hq + h0) * D);
    for (int e = lane; e < G * QW; e += 64) qs[e] = qsrc[e];
    __syncthreads();
    const int32_t* srow = sel + (int64_t)t * g.k;
    for (int it = i0; it < i1; it += 64) {
      const int i = it + lane;
      int64_t row = -1;
      if (i < i1) {
        const int s = list_token(g, L, srow, i);
        if (s >= 0 && s <= qp.p) row = kv_row(g, qp.b, kvh, s);
      }
      QSA_COUNT_ROWS(row >= 0);
      float z[G];
#pragma unroll
      for (int h = 0; h < G; ++h) z[h] = 0.0f;
      if (row >= 0) {
        if constexpr (sizeof(E) == 2) {
          const uint4* kr = reinterpret_cast<const uint4*>(kc + row);
          const uint4* q4 = reinterpret_cast<const uint4*>(qs);
#pragma unroll
          for (int c = 0; c < D / 8; ++c) {
            const uint4 kv = kr[c];
#pragma unroll
            for (int h = 0; h < G; ++h) {
              const uint4 qv = q4[h * (D / 8) + c];
              z[h] = dot2_bf16(kv.x, qv.x, z[h]);
              z[h] = dot2_bf16(kv.y, qv.y, z[h]);
              z[h] = dot2_bf16(kv.z, qv.z, z[h]);
              z[h] = dot2_bf16(kv.w, qv.w, z[h]);
            }
          }
        } else {
          const float4* kr = reinterpret_cast<const float4*>(kc + row);
          const float4* q4 = reinterpret_cast<const float4*>(qs);
#pragma unroll
          for (int c = 0; c < D / 4; ++c) {
            const float4 kv = kr[c];
#pragma unroll
            for (int h = 0; h < G; ++h) {
              const float4 qv = q4[h * (D / 4) + c];
              z[h] = fmaf(kv.x, qv.x, z[h]);
              z[h] = fmaf(kv.y, qv.y, z[h]);
              z[h] = fmaf(kv.z, qv.z, z[h]);
              z[h] = fmaf(kv.w, qv.w, z[h]);
            }
          }
        }
      }
      // Online softmax, base 2; masked lanes contribute 0.
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float zz = (row >= 0) ? z[h] * g.attn_scale_log2 : -INFINITY;
        const float mt = wave_max(zz);
        const float mn = fmaxf(m[h], mt);
        const float alpha = (m[h] == -INFINITY) ? 0.0f : exp2f(m[h] - mn);
        const float p = (zz == -INFINITY) ? 0.0f : exp2f(zz - mn);
        l[h] = l[h] * alpha + wave_sum(p);
#pragma unroll
        for (int d = 0; d < DPL; ++d) o[h][d] *= alpha;
        m[h] = mn;
        ps[lane * G + h] = p;
      }
      rows[lane] = row;
      __syncthreads();
      const int cnt = min(64, i1 - it);
      for (int j = 0; j < cnt; ++j) {
        const int64_t rj = rows[j];
        if (rj < 0) continue;
        float v[DPL];
        if constexpr (sizeof(E) == 2) {
          if constexpr (DPL == 2) {
            const uint32_t vv = reinterpret_cast<const uint32_t*>(vc + rj)[lane];
            v[0] = bf_lo(vv);
            v[1] = bf_hi(vv);
          } else {
            v[0] = to_f32(vc[rj + lane]);
          }
        } else {
#pragma unroll
          for (int d = 0; d < DPL; ++d) v[d] = vc[rj + lane * DPL + d];
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float pj = ps[j * G + h];
#pragma unroll
          for (int d = 0; d < DPL; ++d) o[h][d] = fmaf(pj, v[d], o[h][d]);
        }
      }
      __syncthreads();
    }
  }

  if (plan.n_splits == 1) {
    // Single split: normalise and gate here.
    if (!qp.ok) return;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float inv = l[h] > 0.0f ? 1.0f / l[h] : 0.0f;
#pragma unroll
      for (int d = 0; d < DPL; ++d) {
        const int64_t idx = ((int64_t)t * g.Hq + h0 + h) * D + lane * DPL + d;
        const float gt = to_f32(gate[idx]);
        const float sg = 1.0f / (1.0f + expf(-gt));
        out[idx] = from_f32<E>(o[h][d] * inv * sg);
      }
    }
    return;
  }
  float* P = part + ((int64_t)unit * plan.n_splits + split) * (G * (D + 2));
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int d = 0; d < DPL; ++d) P[h * D + lane * DPL + d] = o[h][d];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      P[G * D + h] = m[h];
      P[G * D + G + h] = qp.ok ? l[h] : -1.0f;  // -1: the query lies outside the capacities
    }
  }
}


// bf16, D = 128 decode kernel.  A workgroup of 4 waves owns one split of one
// (token, KV head) unit; its waves take the split's 64-token tiles in turn.
// Turning list positions into cache rows takes dependent loads (sequence and
// selection entry; position and page; row), so the loads that do not depend
// on each other go out together: the query, n_blocks, the selection entries
// and the sequence search first; then the position and the page-table entries
// of the selected blocks (the tail's pages follow once the position is known).
// Per 64-token tile, in one wave:
//   QK on the matrix cores: S[token][head] = K (A operand: 16 B of a cache row
//     per lane, straight from memory) x Q^T (B operand: the query from LDS,
//     heads padded to 16 columns): 4 token groups x 4 dim steps =
//     16 v_mfma_f32_16x16x32_bf16;
//   online softmax in base 2 on the accumulator layout (a lane holds one head
//     for 16 tokens: in-lane max, then two cross-row exchanges); p rounded to
//     bf16 (the denominator sums the same rounded values) and kept in
//     registers;
//   PV on the matrix cores: p is the A operand as it sits in the accumulator
//     layout; V (a lane loads 4 dims of 32 tokens: 8-byte chunks, two full
//     rows per load instruction) goes to LDS in two 32-token phases and comes
//     back as the B operand through transposing reads: 16 MFMAs per tile.
// The next tile's K is requested after this tile's softmax and its V after
// this tile's PV, so each wave keeps a tile of loads in flight while it
// computes (requesting K right after QK, with more in flight, streams slower).  The loads are unconditional (a wave's last look-ahead reads
// nothing useful): conditional loads would keep two copies of the tile
// registers alive.  With BUF (caches under 4 GiB) K and V go through buffer
// resources: masked rows and the last look-ahead read past the end and come
// back zero, without memory traffic.  Otherwise they read row 0 and masked V
// rows are zeroed in registers.  The 4 waves merge in LDS; a unit with several
// splits writes one partial per split, merged by attn_combine_kernel.
// SEL: the top-k selection is made here from the scores (each workgroup of a
// token makes the same selection; the workgroup of split 0, KV head 0 stores
// it in sel / nblk when they are given), instead of being read from sel.
template <int G, bool BUF, bool SEL, bool KV8>
__global__ __launch_bounds__(256, 2) void attn_decode_kernel(
    Geo g, AttnPlan plan, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ nblk, const uint16_t* __restrict__ gate,
    uint16_t* __restrict__ out, float* __restrict__ part, uint32_t kv_bytes,
    const float* __restrict__ scores, int32_t* __restrict__ sel_out,
    int32_t* __restrict__ nblk_out) {
  static_assert(G >= 1 && G <= 16 && 16 % G == 0, "heads per KV head must divide 16");
  constexpr int D = 128;
  constexpr int RR = 1024;       // list positions resolved per round
  constexpr int EPR = RR / 256;  // positions per thread per round
  __shared__ int32_t rowidx[RR];                // cache row index, -1 = masked
  constexpr int VS = 288;                        // LDS row stride (bytes) of the V half tile
  __shared__ uint4 qs[16][17];                  // query: [head, padded to 16][16-byte chunk]
  // One region, two lives: each wave's V half tile (32 rows) during the tile
  // loop, then the waves' O rows for the merge (after a workgroup barrier).
  constexpr int kVH = 32 * VS, kWo = G * D * 4;
  __shared__ __attribute__((aligned(16))) unsigned char tiles[kWaves * (kVH > kWo ? kVH : kWo)];
  float (*wo_all)[G * D] = reinterpret_cast<float (*)[G * D]>(tiles);
  __shared__ float wm[kWaves][G], wl[kWaves][G];

  // Splits run in reverse launch order: the splits that hold an extra tile
  // (the last ones) are launched first, into the workgroup slots whose waves
  // the hardware favours.
  const int unit = blockIdx.x, split = plan.n_splits - 1 - blockIdx.y, tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int c16 = lane & 15, q4 = lane >> 4;    // MFMA column, lane row group
  const int half = lane >> 5, c32 = lane & 31;  // PV: token half, 4-dim chunk
  unsigned char* VH = tiles + wid * kVH;
  const int t = unit / g.Hkv, kvh = unit - t * g.Hkv, h0 = kvh * G;
  const int32_t* srow = sel + (int64_t)t * g.k;
  const int i0 = split_begin(plan, split), i_end = split_begin(plan, split + 1);
  const int sel_end = g.r > 0 ? (g.k << g.log2r) : 0;  // list positions that come from sel
  const int cap_blocks = g.r > 0 ? (g.cap >> g.log2r) : 0;

  __shared__ int32_t sel_lds[SEL ? kPlanMaxK : 1];


  // Step 1 of the row resolution (independent loads).
  {
    const int hq = tid >> 4, ch = tid & 15;
    uint4 qv = hq < G ? *reinterpret_cast<const uint4*>(q + ((int64_t)t * g.Hq + h0 + hq) * D +
                                                        8 * ch)
                      : make_uint4(0u, 0u, 0u, 0u);
    if constexpr (KV8) {
      if (g.rot) {
        // K/V are stored rotated: the query joins them (q' = H q).  16 lanes
        // hold a head, 8 dimensions each: three stages in the lane, four
        // across lanes; rounded back to bf16.
        const uint32_t w4[4] = {qv.x, qv.y, qv.z, qv.w};
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = __uint_as_float(w4[i] << 16);
          x[2 * i + 1] = __uint_as_float(w4[i] & 0xFFFF0000u);
        }
#pragma unroll
        for (int len = 1; len < 8; len <<= 1)
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (!(i & len)) {
              const float a = x[i], b = x[i + len];
              x[i] = a + b;
              x[i + len] = a - b;
            }
#pragma unroll
        for (int dl = 1; dl < 16; dl <<= 1)
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = fwht_cross(x[i], dl, (ch & dl) != 0);
        qv = make_uint4(bf16_rne(x[0]) | (bf16_rne(x[1]) << 16), bf16_rne(x[2]) | (bf16_rne(x[3]) << 16),
                        bf16_rne(x[4]) | (bf16_rne(x[5]) << 16), bf16_rne(x[6]) | (bf16_rne(x[7]) << 16));
      }
    }
    qs[hq][ch] = qv;
  }
  int nk_raw = 0;
  int32_t sv[EPR], pg[EPR];
  auto fetch_sel = [&](int r0) {
#pragma unroll
    for (int j = 0; j < EPR; ++j) sv[j] = -1;
    if (sel_end == 0) return;  // dense layer: no selection
#pragma unroll
    for (int j = 0; j < EPR; ++j) {
      const int i = r0 + tid + 256 * j;
      // (clamped, unconditional loads: a conditional load waits for the last)
      const int slot = min(i, sel_end - 1) >> g.log2r;
      int32_t v;
      if constexpr (SEL) v = sel_lds[max(slot, 0)];
      else v = srow[max(slot, 0)];
      sv[j] = (i < sel_end) ? v : -1;
    }
  };
  uint32_t kr_sel[8];  // SEL: the keys of this thread's candidates [jb_sel, jb_sel + per_sel)
  const int per_sel = SEL ? (g.nbcap + 255) >> 8 : 0;
  const int jb_sel = tid * per_sel;
  if constexpr (SEL) {
    // (unconditional loads at clamped indices; see select_kernel)
    const float* srw = scores + (int64_t)t * g.nbcap;
    const int jlast = max(g.nbcap - 1, 0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = srw[min(jb_sel + e, jlast)];
      kr_sel[e] = (e < per_sel && jb_sel + e < g.nbcap) ? score_key(v) : 0u;
    }
  } else {
    if (g.r > 0) nk_raw = nblk[t];
    fetch_sel(i0);
  }
  const int b = g.one_q ? t : seq_of(g.cu_q, g.B, t);
  // Token of position i if it lies in the selected part of the list, else -1.
  auto spec_token = [&](int i, int blk) -> int {
    if (g.r == 0) return i < g.cap ? i : -1;
    return (i < sel_end && blk >= 0 && blk < cap_blocks) ? (blk << g.log2r) + (i & (g.r - 1))
                                                         : -1;
  };
  auto fetch_pages = [&](int r0) {
    if (g.page_table == nullptr) return;
#pragma unroll
    for (int j = 0; j < EPR; ++j) {
      const int s = spec_token(r0 + tid + 256 * j, sv[j]);
      const int v = g.page_table[(int64_t)b * g.max_pages + (max(s, 0) >> g.log2ps)];
      pg[j] = s >= 0 ? v : -1;
    }
  };
  // Step 2: the position and the speculative pages.
  const int past = g.past_len[b], cu_b = g.one_q ? t : g.cu_q[b];
  if constexpr (!SEL) fetch_pages(i0);
  const int p = past + (t - cu_b);
  const bool ok = p >= 0 && p < g.cap;
  if constexpr (SEL) {
    // The selection over the candidate blocks 0 .. nb-1 (all of them when
    // there are at most k).
    const int nb = ok ? min((p + 1) >> g.log2r, g.nbcap) : 0;
    nk_raw = min(g.k, nb);
    if (nb <= g.k) {
      for (int i = tid; i < nb; i += 256) sel_lds[i] = i;
    } else {
      block_radix_topk(kr_sel, jb_sel, max(0, min(per_sel, nb - jb_sel)), g.k, sel_lds);
    }
    __syncthreads();
    if (sel_out != nullptr && blockIdx.y == 0 && kvh == 0) {
      for (int i = tid; i < g.k; i += 256) sel_out[(int64_t)t * g.k + i] = i < nk_raw ? sel_lds[i] : -1;
      if (tid == 0 && nblk_out != nullptr) nblk_out[t] = nk_raw;
    }
    fetch_sel(i0);
    fetch_pages(i0);
  }
  ListInfo L = {0, 0, 0, 0};
  if (ok) {
    const int n = p + 1;
    if (g.r == 0) {
      L.n_list = n;
    } else {
      L.nb = n >> g.log2r;
      const int nk = max(0, min(nk_raw, min(g.k, L.nb)));
      L.nsel_tok = nk << g.log2r;
      L.tail0 = L.nb << g.log2r;
      L.n_list = L.nsel_tok + (n - L.tail0);
    }
  }
  const int i1 = min(i_end, L.n_list);
  // Step 3: rows (tail pages looked up now).
  auto resolve_round = [&](int r0) {
#pragma unroll
    for (int j = 0; j < EPR; ++j) {
      const int e = tid + 256 * j, i = r0 + e;
      int s = -1;
      bool spec = false;
      if (i < i1) {
        if (g.r == 0) {
          s = i;
          spec = true;
        } else if (i < L.nsel_tok) {
          const int blk = sv[j];
          if (blk >= 0 && blk < L.nb) {
            s = (blk << g.log2r) + (i & (g.r - 1));
            spec = true;
          }
        } else {
          s = L.tail0 + (i - L.nsel_tok);
        }
      }
      int32_t row = -1;
      if (s >= 0 && s <= p) {
        if (g.page_table == nullptr) {
          row = (int32_t)((int64_t)(b * g.Hkv + kvh) * g.cap + s);
        } else {
          const int page = spec ? pg[j] : g.page_table[(int64_t)b * g.max_pages + (s >> g.log2ps)];
          if (page >= 0 && page < g.n_pages)
            row = (int32_t)(((int64_t)page * g.Hkv + kvh) * g.page_size + (s & (g.page_size - 1)));
        }
      }
      rowidx[e] = row;
    }
  };

  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(kc, kv_bytes), vrs = buffer_rsrc(vc, kv_bytes);
  float m = -INFINITY, lp = 0.0f;  // this lane's head (c16): running max, partial denominator
  // O[head][dim] in the MFMA accumulator layout: O[n][r] = head 4 q4 + r, dim 16 n + c16.
  f32x4_t O[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) O[n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  for (int r0 = i0; r0 < i1; r0 += RR) {
    __syncthreads();  // the previous round's rows are no longer read
    resolve_round(r0);
    __syncthreads();  // rows (and, the first time, the query) visible
    // The next round's selection entries and pages are requested now, so
    // their latency hides behind this round's tiles.
    if (r0 + RR < i1) {
      fetch_sel(r0 + RR);
      fetch_pages(r0 + RR);
    }
    const int r1 = min(r0 + RR, i1);
    uint4 kr[4][4];          // [token group][dim step]: A operands
    uint2 vr[32];            // tokens 32*half + j, dims 4*c32 .. +3
    // 8-bit storage: a lane's 32 contiguous bytes of a K row (dims 32*q4 ..
    // +31; the MFMA k-slots are permuted to match, the query too), and 4
    // bytes of a V row (dims 4*c32 .. +3) per token.
    uint4 k8[4][2];
    uint32_t v8[32];
    uint32_t vmask = 0u;     // without BUF: bit j set = V row of token 32*half + j valid
    // at < 0: no tile.
    auto load_k = [&](int at) {
      const int32_t none = at >= 0 ? 0 : -1;
      const int32_t* rr = rowidx + (at >= 0 ? at - r0 : 0);
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int32_t rj = rr[16 * gi + c16] | none;
        if constexpr (KV8) {
          if constexpr (BUF) {
            const uint32_t off = rj >= 0 ? (uint32_t)rj * D + 32u * q4 : kOobOffset;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
              k8[gi][hh] = __builtin_bit_cast(
                  uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 16 * hh, kStreamPolicy));
          } else {
            const uint8_t* src = reinterpret_cast<const uint8_t*>(kc) + (int64_t)max(rj, 0) * D + 32 * q4;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
              k8[gi][hh] = __builtin_bit_cast(
                  uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + 16 * hh)));
          }
        } else if constexpr (BUF) {
          const uint32_t off = rj >= 0 ? (uint32_t)rj * (D * 2) + 16u * q4 : kOobOffset;
#pragma unroll
          for (int db = 0; db < 4; ++db)
            kr[gi][db] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 64 * db, kStreamPolicy));
        } else {
          const uint16_t* src = kc + (int64_t)max(rj, 0) * D + 8 * q4;
#pragma unroll
          for (int db = 0; db < 4; ++db)
            kr[gi][db] = __builtin_bit_cast(
                uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + 32 * db)));
        }
      }
    };
    auto load_v = [&](int at) {
      const int32_t none = at >= 0 ? 0 : -1;
      const int32_t* rr = rowidx + (at >= 0 ? at - r0 : 0) + half;
      uint32_t vm = 0u;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int32_t rj = rr[2 * j] | none;  // token 2 j + half
        if constexpr (KV8) {
          if constexpr (BUF) {
            const uint32_t off = rj >= 0 ? (uint32_t)rj * D + 4u * c32 : kOobOffset;
            v8[j] = __builtin_amdgcn_raw_buffer_load_b32(vrs, off, 0, kStreamPolicy);
          } else {
            v8[j] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(
                reinterpret_cast<const uint8_t*>(vc) + (int64_t)max(rj, 0) * D + 4 * c32));
            vm |= (rj >= 0 ? 1u : 0u) << j;
          }
        } else if constexpr (BUF) {
          const uint32_t off = rj >= 0 ? (uint32_t)rj * (D * 2) + 8u * c32 : kOobOffset;
          vr[j] = __builtin_bit_cast(
              uint2, __builtin_amdgcn_raw_buffer_load_b64(vrs, off, 0, kStreamPolicy));
        } else {
          vr[j] = __builtin_bit_cast(uint2, __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(
                                                vc + (int64_t)max(rj, 0) * D + 4 * c32)));
          vm |= (rj >= 0 ? 1u : 0u) << j;
        }
      }
      vmask = vm;
    };
    int it = r0 + 64 * wid;
    if (it < r1) {
      load_k(it);
      load_v(it);
      for (;;) {
        const int nit = it + 64 * kWaves;
        const bool has_next = nit < r1;
        const int32_t* rows = rowidx + (it - r0);
        QSA_COUNT_ROWS(rows[lane] >= 0);
        const bool full = __all(rows[lane] >= 0);

        uint4 qb[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) qb[db] = qs[c16][KV8 ? 4 * q4 + db : 4 * db + q4];
        f32x4_t z[4];
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          z[gi] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            uint4 a;
            if constexpr (KV8) {  // 8 codes -> 8 bf16 (exact)
              const uint4 h = k8[gi][db >> 1];
              const uint32_t w0 = (db & 1) ? h.z : h.x, w1 = (db & 1) ? h.w : h.y;
              a = make_uint4(
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true)));
            } else {
              a = kr[gi][db];
            }
            z[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, qb[db]), z[gi], 0,
                0, 0);
          }
        }

        // Lane holds head c16 for tokens 16*gi + 4*q4 + e.
        float tmax = -INFINITY;
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float v = z[gi][e] * g.attn_scale_log2;
            if (!full && rows[16 * gi + 4 * q4 + e] < 0) v = -INFINITY;
            z[gi][e] = v;
            tmax = fmaxf(tmax, v);
          }
        tmax = max_xor32(max_xor16(tmax));
        const float mn = fmaxf(m, tmax);
        const float alpha = (m == -INFINITY) ? 0.0f : exp2f(m - mn);
        m = mn;
        float psum = 0.0f;
        uint32_t pw[4][2];  // p as bf16 pairs: tokens 16 gi + 4 q4 + (0, 1) and (2, 3)
        const float mb = mn == -INFINITY ? 0.0f : mn;  // while mn is -inf, so is every z
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            // exp2(-inf) = 0; hardware round-to-nearest-even to bf16
            const uint32_t pa = __builtin_bit_cast(uint16_t, (__bf16)exp2f(z[gi][2 * pr] - mb));
            const uint32_t pc = __builtin_bit_cast(uint16_t, (__bf16)exp2f(z[gi][2 * pr + 1] - mb));
            psum += bf_lo(pa) + bf_lo(pc);
            pw[gi][pr] = pa | (pc << 16);
          }
        lp = fmaf(lp, alpha, psum);
        // Lane (dim, q4) holds the O rows of heads 4 q4 + r: their factors.
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ah =
              __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (4 * q4 + r), __float_as_int(alpha)));
#pragma unroll
          for (int n = 0; n < 8; ++n) O[n][r] *= ah;
        }

        // The next tile's K is requested only now, after the softmax: fewer
        // requests in flight at once stream faster on this memory system.
        __builtin_amdgcn_sched_barrier(0);
        load_k(has_next ? nit : -1);
        __builtin_amdgcn_sched_barrier(0);
        // O += P V on the matrix cores, in two phases of 32 tokens.  P is the
        // A operand straight from the softmax registers: phase ph pairs tokens
        // 32 ph + 4 q4 + (0..3) and 32 ph + 16 + 4 q4 + (0..3) (the order of the
        // tokens inside a tile is free as long as V follows it).  V: this lane
        // holds tokens 2 j + half (dims 4 c32 ..); a phase's 32 rows go to VH
        // row-major, and the B operand (dim 16 n + c16, the same 8 tokens) comes
        // back through two transposing reads (ds_read_b64_tr_b16: inside a
        // 16-lane group, element j of lane i is element i % 4 of the 8 bytes
        // that lane 4 j + i / 4 addresses).
        typedef short v4s __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int ph = 0; ph < 2; ++ph) {
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            const int j = 16 * ph + jj;
            uint2 v2;
            if constexpr (KV8) {  // 4 codes -> 4 bf16 (exact), masked rows zeroed first
              uint32_t a8 = v8[j];
              if constexpr (!BUF) a8 &= ((vmask >> j) & 1u) ? ~0u : 0u;
              v2 = make_uint2(
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a8, 1.0f, false)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a8, 1.0f, true)));
            } else {
              v2 = vr[j];
              if constexpr (!BUF) {
                const uint32_t km = ((vmask >> j) & 1u) ? ~0u : 0u;
                v2.x &= km;
                v2.y &= km;
              }
            }
            *reinterpret_cast<uint2*>(VH + (2 * jj + half) * VS + 8 * c32) = v2;
          }
          wave_sync();
          const uint4 pa = make_uint4(pw[2 * ph][0], pw[2 * ph][1], pw[2 * ph + 1][0], pw[2 * ph + 1][1]);
          const unsigned char* v0 = VH + (4 * q4 + (c16 >> 2)) * VS + 8 * (c16 & 3);
#pragma unroll
          for (int n = 0; n < 8; ++n) {
            const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s*)(v0 + 32 * n));
            const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s*)(v0 + 16 * VS + 32 * n));
            const uint4 vb = make_uint4(__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                                        __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y);
            O[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, pa),
                                                           __builtin_bit_cast(bf16x8_t, vb), O[n], 0, 0, 0);
          }
          wave_sync();  // VH is rewritten by the next phase or tile
        }
        __builtin_amdgcn_sched_barrier(0);
        load_v(has_next ? nit : -1);
        __builtin_amdgcn_sched_barrier(0);
        wave_sync();
        if (!has_next) break;
        it = nit;
      }
    }
  }

  // Wave totals: l over the four lane rows of a head; O rows per head (once
  // every wave is past its tile loop: the rows overlay the V tiles).
  const float lt = sum_xor32(sum_xor16(lp));
  __syncthreads();
  if (lane < G) {
    wm[wid][lane] = m;
    wl[wid][lane] = lt;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * q4 + r;
    if (h < G) {
#pragma unroll
      for (int n = 0; n < 8; ++n) wo_all[wid][h * D + 16 * n + c16] = O[n][r];
    }
  }
  __syncthreads();

  // Merge the 4 waves: thread -> EPT consecutive elements of one head.
  constexpr int EPT = (G * D >= 256) ? G * D / 256 : 1;
  const bool has_elem = tid * EPT < G * D;
  const int e0 = has_elem ? tid * EPT : 0, hh = e0 / D, d0 = e0 - hh * D;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wm[w][hh]);
  float Lw = 0.0f, Ow[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) Ow[i] = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float mw = wm[w][hh];
    const float a = (mw == -INFINITY) ? 0.0f : exp2f(mw - M);
    Lw = fmaf(wl[w][hh], a, Lw);
    const float* src = wo_all[w] + hh * D + d0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) Ow[i] = fmaf(src[i], a, Ow[i]);
  }

  if (plan.n_splits == 1) {
    if (!ok) return;
    const float inv = Lw > 0.0f ? 1.0f / Lw : 0.0f;
    float Of[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) Of[i] = Ow[i] * inv;
    if constexpr (KV8) kv8_output(g, Of, d0 / EPT);
    if (!has_elem) return;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int64_t idx = ((int64_t)t * g.Hq + h0 + hh) * D + d0 + i;
      const float sg = 1.0f / (1.0f + expf(-to_f32(gate[idx])));
      out[idx] = from_f32<uint16_t>(Of[i] * sg);
    }
    return;
  }
  constexpr int SP = G * (D + 2);
  float* P = part + ((int64_t)unit * plan.n_splits + split) * SP;
  if (has_elem) {
#pragma unroll
    for (int i = 0; i < EPT; ++i) P[hh * D + d0 + i] = Ow[i];
  }
  if (has_elem && d0 == 0) {
    P[G * D + hh] = M;
    P[G * D + G + hh] = ok ? Lw : -1.0f;  // -1: the query lies outside the capacities
  }
}

// ---------------------------------------------------------------------------
// Prefill attention on MFMA (bf16, D = 128): one wave per (token, KV head)
// unit, 4 units per workgroup, no splits (prefill has units to spare).
// Matrix-core layout of v_mfma_f32_16x16x32_bf16 (64 lanes, l = lane):
//   A[i][k]: i = l%16, k = 8*(l/16) + e;  B[k][j]: j = l%16, k = 8*(l/16) + e;
//   C[i][j]: j = l%16, i = 4*(l/16) + r.
// Per 64-key tile of the unit's selection list (lane l = (c16, grp)):
//   S^T[key][head] = K (A: key 16n + c16) x Q^T (B: head c16, zero past G):
//       4 key tiles x 4 k-steps = 16 MFMAs; lane (c16, grp) then holds head
//       c16's scores of keys 16n + 4 grp + r;
//   online softmax in base 2: a head's 64 scores sit in the 4 lanes c16 + 16 g
//       (in-lane maximum over 16, then two row swaps);
//   P feeds P x V as the A operand straight from those registers: k-step ks
//       takes keys 16 (2 ks) + 4 grp + r, then 16 (2 ks + 1) + 4 grp + r (the
//       order of the keys inside a tile is free as long as V follows it);
//   V goes to LDS row-major as loaded; its B operand (dim 16n + c16, the same
//       8 keys) comes back through two transposing reads (ds_read_b64_tr_b16:
//       inside a 16-lane group, element j of lane i is element i % 4 of the 8
//       bytes that lane 4 j + i / 4 addresses);
//   O[head][dim] += P x V, 8 dim tiles x 2 k-steps; each head's rescale
//       factor reaches the lanes holding its O rows through ds_bpermute.
// K and V are loaded coalesced (the 4 lanes of a quad read 64 contiguous
// bytes of one row) and both requested before the first MFMA; K reaches the
// A-operand layout through ds_bpermute.  V rows are 288 B apart in LDS, so the
// 4 rows one 16-lane transposing read touches fall on distinct banks.
template <int G>
__global__ __launch_bounds__(256, 2) void attn_prefill_mfma_kernel(
    Geo g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ nblk, const uint16_t* __restrict__ gate,
    uint16_t* __restrict__ out) {
  static_assert(G <= 16, "heads per KV head must fit the 16 MFMA columns");
  constexpr int D = 128;
  constexpr int VS = 288;                 // LDS row stride (bytes) of the V tile
  constexpr int RND = 128;                // list positions resolved per round
  typedef short v4s __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) unsigned char V_all[kWaves][64 * VS];
  __shared__ __attribute__((aligned(16))) int32_t rows_all[kWaves][RND];
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int t, kvh;
  if (8 % g.Hkv == 0) {
    // Workgroups are dispatched round-robin over the 8 XCDs (blockIdx % 8):
    // XCD x serves KV head x / (8 / Hkv), so that its L2 holds the K/V rows of
    // one head only; consecutive workgroups of an XCD take consecutive tokens.
    const int per = 8 / g.Hkv, x = blockIdx.x & 7;
    kvh = x / per;
    t = ((blockIdx.x >> 3) * per + (x - kvh * per)) * kWaves + wid;
    if (t >= g.T) return;  // whole wave; only wave-level sync below
  } else {
    const int unit = blockIdx.x * kWaves + wid;
    if (unit >= g.T * g.Hkv) return;
    t = unit / g.Hkv;
    kvh = unit - t * g.Hkv;
  }
  unsigned char* Vl = V_all[wid];
  int32_t* rows = rows_all[wid];
  const QueryPos qp = query_pos(g, t);
  if (!qp.ok) return;
  const ListInfo L = list_info(g, qp, nblk, t);
  const int32_t* srow = sel + (int64_t)t * g.k;
  const int h0 = kvh * G;
  const int c16 = lane & 15, grp = lane >> 4;
  const int kq = lane >> 2, cq = lane & 3;  // coalesced loads: row, 16-byte chunk

  // Q^T as the B operand: column c16 = head (zero past G), k = dims 32 ks + 8 grp + e.
  bf16x8_t qa[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (c16 < G)
      w = *reinterpret_cast<const uint4*>(q + ((int64_t)t * g.Hq + h0 + c16) * D + 32 * ks + 8 * grp);
    qa[ks] = __builtin_bit_cast(bf16x8_t, w);
  }
  float m = -INFINITY;  // head c16: running maximum (base 2)
  float ls = 0.0f;      // head c16: this lane's share of the denominator
  f32x4_t O[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) O[n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Selection entries of a round's list positions, requested one round ahead
  // so that their latency hides behind the previous round's tiles.
  int32_t se[RND / 64];
  auto fetch_sel = [&](int r0) {
#pragma unroll
    for (int e = 0; e < RND / 64; ++e) {
      const int i = r0 + 64 * e + lane;
      se[e] = (g.r > 0 && i < L.nsel_tok) ? srow[i >> g.log2r] : -1;
    }
  };
  fetch_sel(0);
  for (int r0 = 0; r0 < L.n_list; r0 += RND) {
    // Resolve this round's cache rows (list order: selected blocks, then the tail).
#pragma unroll
    for (int e = 0; e < RND / 64; ++e) {
      const int i = r0 + 64 * e + lane;
      int32_t rv = -1;
      if (i < L.n_list) {
        int s;
        if (g.r == 0) s = i;
        else if (i < L.nsel_tok) s = (se[e] >= 0 && se[e] < L.nb) ? (se[e] << g.log2r) + (i & (g.r - 1)) : -1;
        else s = L.tail0 + (i - L.nsel_tok);
        const int64_t rr = (s >= 0 && s <= qp.p) ? kv_row(g, qp.b, kvh, s) : -1;
        rv = rr >= 0 ? (int32_t)(rr / D) : -1;
      }
      rows[64 * e + lane] = rv;
    }
    fetch_sel(r0 + RND);
    wave_sync();
    const int r1 = min(r0 + RND, L.n_list);
    for (int it = r0; it < r1; it += 64) {
      const int32_t* tr = rows + (it - r0);
      QSA_COUNT_ROWS(it + lane < r1 && tr[lane] >= 0);
      // K: load n, k-step ks holds row 16n + kq, bytes 16 cq + 64 ks.
      // V: rows 4 kq + s, bytes 16 (cq + 4 j).
      int32_t klr[4], vrow[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) klr[n] = tr[16 * n + kq];
#pragma unroll
      for (int sft = 0; sft < 4; ++sft) vrow[sft] = tr[4 * kq + sft];
      uint4 kl[4][4], vv[4][4];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int64_t base = (int64_t)(klr[n] >= 0 ? klr[n] : 0) * D + 8 * cq;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          kl[n][ks] = *reinterpret_cast<const uint4*>(kc + base + 32 * ks);
      }
#pragma unroll
      for (int sft = 0; sft < 4; ++sft) {
        const bool ok = vrow[sft] >= 0;
        const int64_t base = (int64_t)(ok ? vrow[sft] : 0) * D;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 w = *reinterpret_cast<const uint4*>(vc + base + 8 * (cq + 4 * j));
          vv[j][sft] = ok ? w : make_uint4(0u, 0u, 0u, 0u);
        }
      }
      // V -> LDS as loaded.
#pragma unroll
      for (int sft = 0; sft < 4; ++sft)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint4*>(Vl + (4 * kq + sft) * VS + 16 * (cq + 4 * j)) = vv[j][sft];
      // K to the A-operand layout: lane (c16, grp) takes the chunk lane 4 c16 + grp loaded.
      const int src = 4 * (4 * c16 + grp);
      f32x4_t S[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        S[n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          S[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, lane_gather(kl[n][ks], src)), qa[ks], S[n], 0, 0, 0);
      }
      // Online softmax of head c16 over this lane's keys 16n + 4 grp + r.
      int4 kv[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) kv[n] = *reinterpret_cast<const int4*>(tr + 16 * n + 4 * grp);
      float mx = -INFINITY;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int vr[4] = {kv[n].x, kv[n].y, kv[n].z, kv[n].w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float z = vr[r] >= 0 ? S[n][r] * g.attn_scale_log2 : -INFINITY;
          S[n][r] = z;
          mx = fmaxf(mx, z);
        }
      }
      mx = max_xor32(max_xor16(mx));
      const float mn = fmaxf(m, mx);
      const float alpha = (m == -INFINITY) ? 0.0f : exp2f(m - mn);
      m = mn;
      const float mb = mn == -INFINITY ? 0.0f : mn;  // while mn is -inf, so is every z
      uint32_t pw[4][2];  // bf16 pairs: keys (r 0, 1) and (r 2, 3) of key tile n
      float lsum = 0.0f;
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          // exp2(-inf) = 0; hardware round-to-nearest-even to bf16
          const uint16_t p0 = __builtin_bit_cast(uint16_t, (__bf16)exp2f(S[n][2 * h] - mb));
          const uint16_t p1 = __builtin_bit_cast(uint16_t, (__bf16)exp2f(S[n][2 * h + 1] - mb));
          lsum += to_f32(p0) + to_f32(p1);
          pw[n][h] = (uint32_t)p0 | ((uint32_t)p1 << 16);
        }
      ls = fmaf(ls, alpha, lsum);
      // Lane (dim, grp) holds O rows of heads 4 grp + r: their factors.
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (4 * grp + r), __float_as_int(alpha)));
#pragma unroll
        for (int n = 0; n < 8; ++n) O[n][r] *= a;
      }
      wave_sync();  // the V tile is in LDS
      // O += P V: k-step ks pairs P's keys 32 ks + 4 grp + (0..3, 16..19)
      // with two transposing reads of V rows 32 ks + 4 grp + c16 / 4 (+16).
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint4 pa = make_uint4(pw[2 * ks][0], pw[2 * ks][1], pw[2 * ks + 1][0], pw[2 * ks + 1][1]);
        const unsigned char* vrow0 = Vl + (32 * ks + 4 * grp + (c16 >> 2)) * VS + 8 * (c16 & 3);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4s*)(vrow0 + 32 * n));
          const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4s*)(vrow0 + 16 * VS + 32 * n));
          const uint4 vb = make_uint4(__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                                      __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y);
          O[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, pa),
                                                         __builtin_bit_cast(bf16x8_t, vb), O[n], 0, 0, 0);
        }
      }
      wave_sync();  // the next tile may overwrite V
    }
    wave_sync();
  }
  // Denominator of head c16 (its 4 lanes), then to the lanes of its O rows.
  float l = sum_xor32(sum_xor16(ls));
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float lr = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (4 * grp + r), __float_as_int(l)));
    const int h = 4 * grp + r;
    if (h >= G) continue;
    const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int64_t idx = ((int64_t)t * g.Hq + h0 + h) * D + 16 * n + c16;
      const float sg = 1.0f / (1.0f + expf(-to_f32(gate[idx])));
      out[idx] = bf16_rne(O[n][r] * inv * sg);
    }
  }
}

template <typename E, int G, int D>
hipError_t attend_impl(const Geo& g, const AttnPlan& plan, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* sel, const int32_t* n_blocks,
                       const void* gate, void* out, float* part, const InKernelSelect& fs,
                       hipStream_t st) {
  const float* scores = fs.scores;
  int32_t* sel_out = fs.sel_out;
  int32_t* nblk_out = fs.n_blocks_out;
  if constexpr (sizeof(E) == 2 && D == 128) {
    if (plan.mfma) {
      // 8 % Hkv == 0: 8 workgroups (one per XCD) per 8 / Hkv groups of kWaves tokens.
      const int tg = (g.T + kWaves - 1) / kWaves;
      const int blocks = (8 % g.Hkv == 0) ? 8 * ((tg + 8 / g.Hkv - 1) / (8 / g.Hkv))
                                          : (g.T * g.Hkv + kWaves - 1) / kWaves;
      attn_prefill_mfma_kernel<G><<<blocks, 64 * kWaves, 0, st>>>(
          g, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
          static_cast<const uint16_t*>(v_cache), sel, n_blocks,
          static_cast<const uint16_t*>(gate), static_cast<uint16_t*>(out));
      return hipGetLastError();
    }
  }
  dim3 grid(g.T * g.Hkv, plan.n_splits);
  if constexpr (sizeof(E) == 2 && D == 128) {
    const int64_t rows = g.page_table ? (int64_t)g.n_pages * g.Hkv * g.page_size
                                      : (int64_t)g.B * g.Hkv * g.cap;
    const int64_t bytes = rows * D * g.kv_esz;
    auto launch = [&](auto buf, auto fused, auto kv8) {
      attn_decode_kernel<G, decltype(buf)::value, decltype(fused)::value, decltype(kv8)::value>
          <<<grid, 64 * kWaves, 0, st>>>(
              g, plan, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
              static_cast<const uint16_t*>(v_cache), sel, n_blocks,
              static_cast<const uint16_t*>(gate), static_cast<uint16_t*>(out), part,
              decltype(buf)::value ? (uint32_t)bytes : 0u, scores, sel_out, nblk_out);
    };
    const bool buf = bytes < (int64_t)kOobOffset;
    auto launch_kv = [&](auto kv8) {
      if (scores != nullptr) {
        if (buf) launch(std::true_type{}, std::true_type{}, kv8);
        else launch(std::false_type{}, std::true_type{}, kv8);
      } else {
        if (buf) launch(std::true_type{}, std::false_type{}, kv8);
        else launch(std::false_type{}, std::false_type{}, kv8);
      }
    };
    if (g.kv8) launch_kv(std::true_type{});
    else launch_kv(std::false_type{});
  } else {
    attn_split_kernel<E, G, D><<<grid, 64, 0, st>>>(
        g, plan, static_cast<const E*>(q), static_cast<const E*>(k_cache),
        static_cast<const E*>(v_cache), sel, n_blocks, static_cast<const E*>(gate),
        static_cast<E*>(out), part);
  }
  if (plan.n_splits > 1) {
    attn_combine_kernel<E, G, D><<<g.T * g.Hkv, 256, 0, st>>>(
        g, plan, part, static_cast<const E*>(gate), static_cast<E*>(out));
  }
  return hipGetLastError();
}

template <typename E, int G>
hipError_t attend_d(const Geo& g, const AttnPlan& plan, const void* q, const void* kc,
                    const void* vc, const int32_t* sel, const int32_t* nb, const void* gate,
                    void* out, float* part, const InKernelSelect& fs, hipStream_t st) {
  if (g.D == 64) return attend_impl<E, G, 64>(g, plan, q, kc, vc, sel, nb, gate, out, part, fs, st);
  return attend_impl<E, G, 128>(g, plan, q, kc, vc, sel, nb, gate, out, part, fs, st);
}

template <typename E>
hipError_t attend_g(const Geo& g, const AttnPlan& plan, const void* q, const void* kc,
                    const void* vc, const int32_t* sel, const int32_t* nb, const void* gate,
                    void* out, float* part, const InKernelSelect& fs, hipStream_t st) {
  switch (g.G) {
    case 1: return attend_d<E, 1>(g, plan, q, kc, vc, sel, nb, gate, out, part, fs, st);
    case 2: return attend_d<E, 2>(g, plan, q, kc, vc, sel, nb, gate, out, part, fs, st);
    case 4: return attend_d<E, 4>(g, plan, q, kc, vc, sel, nb, gate, out, part, fs, st);
    case 8: return attend_d<E, 8>(g, plan, q, kc, vc, sel, nb, gate, out, part, fs, st);
    default: return attend_d<E, 16>(g, plan, q, kc, vc, sel, nb, gate, out, part, fs, st);
  }
}

// The many-token scorer's grid: as many workgroups as the GPU holds at once
// (from the kernel's occupancy, once per instantiation), or fewer when there
// are fewer units than waves.
template <typename E, int HIM, int DI>
void score_tile_launch(const Geo& g, const E* q, const float* w, const float* pooled,
                       float* scores, hipStream_t st) {
  static const int resident = [] {
    int dev = 0, per_cu = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, score_tile_kernel<E, HIM, DI>, 256,
                                                     0) != hipSuccess ||
        per_cu < 1)
      return 1024;
    return per_cu * prop.multiProcessorCount;
  }();
  const int64_t units = (int64_t)g.T * std::max(1, (g.nbcap + 63) / 64);
  const int64_t wgs = std::min<int64_t>(resident, (units + 3) / 4);
  score_tile_kernel<E, HIM, DI><<<(unsigned)wgs, 256, 0, st>>>(g, q, w, pooled, scores);
}

template <typename E, int DI, int MODE>
void score_hd(const Geo& g, const void* qI, const float* w, float* pooled, float* scores,
              const AppendArgs& ap, const RopeTab& rt, hipStream_t st) {
  // (decode form: two more workgroups per token, the appender and the pooler)
  dim3 grid(g.T, std::max(1, (g.nbcap + 63) / 64) + (MODE != 0 ? 2 : 0));
  const E* q = static_cast<const E*>(qI);
  const E* kn = static_cast<const E*>(ap.k_new);
  const E* vn = static_cast<const E*>(ap.v_new);
  const E* in = static_cast<const E*>(ap.kI_new);
  E* kc = static_cast<E*>(ap.k_cache);
  E* vc = static_cast<E*>(ap.v_cache);
  E* ic = static_cast<E*>(ap.kI_cache);
  if constexpr (MODE == 0) {
    if (g.HI <= 4) score_tile_launch<E, 4, DI>(g, q, w, pooled, scores, st);
    else if (g.HI <= 8) score_tile_launch<E, 8, DI>(g, q, w, pooled, scores, st);
    else score_tile_launch<E, 16, DI>(g, q, w, pooled, scores, st);
  } else if (g.HI <= 4) {
    score_kernel<E, 4, DI, MODE><<<grid, 64, 0, st>>>(g, q, w, pooled, scores, kn, vn, in, kc, vc, ic, rt);
  } else if (g.HI <= 8) {
    score_kernel<E, 8, DI, MODE><<<grid, 64, 0, st>>>(g, q, w, pooled, scores, kn, vn, in, kc, vc, ic, rt);
  } else {
    score_kernel<E, 16, DI, MODE><<<grid, 64, 0, st>>>(g, q, w, pooled, scores, kn, vn, in, kc, vc, ic, rt);
  }
}

template <typename E, int MODE>
hipError_t score_h(const Geo& g, const void* qI, const float* w, float* pooled, float* scores,
                   const AppendArgs& ap, const RopeTab& rt, hipStream_t st) {
  if (g.dI == 32) score_hd<E, 32, MODE>(g, qI, w, pooled, scores, ap, rt, st);
  else if (g.dI == 64) score_hd<E, 64, MODE>(g, qI, w, pooled, scores, ap, rt, st);
  else score_hd<E, 128, MODE>(g, qI, w, pooled, scores, ap, rt, st);
  return hipGetLastError();
}

}  // namespace

#ifdef QSA_COUNT_KEYS
hipError_t keys_visited(unsigned long long* value, bool reset) {
  hipError_t e = hipMemcpyFromSymbol(value, HIP_SYMBOL(g_keys_visited), sizeof(*value));
  if (e != hipSuccess || !reset) return e;
  const unsigned long long zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_keys_visited), &zero, sizeof(zero));
}
#endif

bool attend_supported(int G, int D) {
  return (G == 1 || G == 2 || G == 4 || G == 8 || G == 16) && (D == 64 || D == 128);
}

hipError_t launch_append_pool(const Geo& g, int elem, const void* k_new, const void* v_new,
                              const void* kI_new, void* k_cache, void* v_cache, void* kI_cache,
                              float* pooled, const RopeTab& idx_rope, hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  if (elem == kBF16) {
    append_pool_kernel<uint16_t><<<dim3(g.T, 2), 256, 0, st>>>(
        g, static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
        static_cast<const uint16_t*>(kI_new), static_cast<uint16_t*>(k_cache),
        static_cast<uint16_t*>(v_cache), static_cast<uint16_t*>(kI_cache), pooled, idx_rope);
  } else {
    append_pool_kernel<float><<<dim3(g.T, 2), 256, 0, st>>>(
        g, static_cast<const float*>(k_new), static_cast<const float*>(v_new),
        static_cast<const float*>(kI_new), static_cast<float*>(k_cache),
        static_cast<float*>(v_cache), static_cast<float*>(kI_cache), pooled, idx_rope);
  }
  return hipGetLastError();
}

hipError_t launch_score(const Geo& g, int elem, const void* qI, const float* w, float* pooled,
                        float* scores, hipStream_t st) {
  if (g.T == 0 || g.nbcap == 0) return hipSuccess;
  const AppendArgs none = {};
  const RopeTab no_rope = {};
  return elem == kBF16 ? score_h<uint16_t, 0>(g, qI, w, pooled, scores, none, no_rope, st)
                       : score_h<float, 0>(g, qI, w, pooled, scores, none, no_rope, st);
}

hipError_t launch_score_append(const Geo& g, int elem, const void* qI, const float* w,
                               float* pooled, float* scores, const AppendArgs& ap,
                               const RopeTab& idx_rope, hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  return elem == kBF16 ? score_h<uint16_t, 1>(g, qI, w, pooled, scores, ap, idx_rope, st)
                       : score_h<float, 1>(g, qI, w, pooled, scores, ap, idx_rope, st);
}

hipError_t launch_select(const Geo& g, const float* scores, int32_t* sel, int32_t* n_blocks,
                         hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  if (g.nbcap <= kSelectWaveBlocks)
    select_wave_kernel<<<(g.T + 3) / 4, 256, 0, st>>>(g, scores, sel, n_blocks);
  else if (g.nbcap <= kSelectMaxBlocks) select_kernel<<<g.T, 256, 0, st>>>(g, scores, sel, n_blocks);
  else select_large_kernel<<<g.T, 256, 0, st>>>(g, scores, sel, n_blocks);
  return hipGetLastError();
}

hipError_t launch_attend(const Geo& g, int elem, const AttnPlan& plan, const void* q,
                         const void* k_cache, const void* v_cache, const int32_t* sel,
                         const int32_t* n_blocks, const void* gate, void* out, float* part,
                         hipStream_t st, const InKernelSelect& fs) {
  if (g.T == 0) return hipSuccess;
  return elem == kBF16 ? attend_g<uint16_t>(g, plan, q, k_cache, v_cache, sel, n_blocks, gate,
                                            out, part, fs, st)
                       : attend_g<float>(g, plan, q, k_cache, v_cache, sel, n_blocks, gate, out,
                                         part, fs, st);
}

}  // namespace qsa
