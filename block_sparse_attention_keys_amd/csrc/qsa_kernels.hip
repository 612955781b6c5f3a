// QSA hot-path kernels for gfx950 (MI355X): wave64, LDS, dot2 / MFMA.
//
// Kernels (one QSA layer step):
//   append_pool   write new K/V/indexer-key rows at each sequence's past_len and
//                 pool every block the new tokens complete (mean of r indexer
//                 keys, fp32, tokens ascending).
//   score         relu-weighted multi-head block scores, one lane per 4 blocks,
//                 fp32 fmaf chains in a fixed order (the order is what makes the
//                 selection reproducible bit for bit).
//   select        per-query top-k by (score desc, index asc): 4-pass 8-bit radix
//                 select in LDS, then an ascending compaction.
//   attn_split    gated GQA softmax attention over the selected blocks + tail,
//                 split along the selection list; one wave per (token, KV head,
//                 split); online softmax in base 2.
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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
template <typename E> __device__ __forceinline__ E from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) { return bf16_rne(x); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sequence of token t: the largest b with cu_q[b] <= t.
__device__ __forceinline__ int seq_of(const int32_t* cu_q, int B, int t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

struct QueryPos {
  int b, p;
  bool ok;
};
__device__ __forceinline__ QueryPos query_pos(const Geo& g, int t) {
  QueryPos q;
  q.b = seq_of(g.cu_q, g.B, t);
  q.p = g.past_len[q.b] + (t - g.cu_q[q.b]);
  q.ok = q.p >= 0 && q.p < g.cap;
  return q;
}

// Element offset of row s of (sequence b, KV head kvh) in a K or V cache, or -1
// when the row is outside the stated capacity / page pool.
__device__ __forceinline__ int64_t kv_row(const Geo& g, int b, int kvh, int s) {
  if (s < 0 || s >= g.cap) return -1;
  if (g.page_table == nullptr) return ((int64_t)(b * g.Hkv + kvh) * g.cap + s) * g.D;
  const int page = g.page_table[(int64_t)b * g.max_pages + (s >> g.log2ps)];
  if (page < 0 || page >= g.n_pages) return -1;
  return (((int64_t)page * g.Hkv + kvh) * g.page_size + (s & (g.page_size - 1))) * g.D;
}
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
// append + pool: one workgroup per new token.
template <typename E>
__global__ __launch_bounds__(256) void append_pool_kernel(
    Geo g, const E* __restrict__ k_new, const E* __restrict__ v_new,
    const E* __restrict__ kI_new, E* __restrict__ k_cache, E* __restrict__ v_cache,
    E* __restrict__ kI_cache, float* __restrict__ pooled) {
  const int t = blockIdx.x, tid = threadIdx.x;
  const QueryPos qp = query_pos(g, t);
  if (!qp.ok) return;
  constexpr int EPV = 16 / sizeof(E);  // elements per 16-byte copy
  if (k_new != nullptr) {
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
  // The token that ends block j pools it.  Rows appended by this same call are
  // read from kI_new (another workgroup may not have stored them yet); older
  // rows come from the cache.
  if (pooled == nullptr || g.r == 0 || ((qp.p + 1) & (g.r - 1)) != 0) return;
  const int j = qp.p >> g.log2r;
  const int past = g.past_len[qp.b], t0 = g.cu_q[qp.b];
  for (int x = tid; x < g.dI; x += blockDim.x) {
    float acc = 0.0f;
    for (int s = j << g.log2r; s <= qp.p; ++s) {
      float v = 0.0f;
      if (s >= past) {
        v = to_f32(kI_new[(int64_t)(t0 + s - past) * g.dI + x]);
      } else {
        const int64_t row = idx_row(g, qp.b, s);
        if (row >= 0) v = to_f32(kI_cache[row + x]);
      }
      acc = acc + v;
    }
    pooled[((int64_t)qp.b * g.dI + x) * g.pooled_ld + j] = acc * g.inv_r;
  }
}

// ---------------------------------------------------------------------------
// score: grid (T, ceil(nbcap/256)), one wave; lane owns blocks j0..j0+3.
template <typename E, int HIM>
__global__ __launch_bounds__(64) void score_kernel(Geo g, const E* __restrict__ qI,
                                                   const float* __restrict__ w,
                                                   const float* __restrict__ pooled,
                                                   float* __restrict__ scores) {
  __shared__ float qT[128 * HIM];  // [x][h]
  __shared__ float wsh[HIM];
  const int t = blockIdx.x, lane = threadIdx.x;
  const QueryPos qp = query_pos(g, t);
  const int nb = qp.ok ? ((qp.p + 1) >> g.log2r) : 0;
  const int j0 = blockIdx.y * 256 + lane * 4;
  float* srow = scores + (int64_t)t * g.nbcap;
  float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if ((int)blockIdx.y * 256 < nb) {
    const int HI = g.HI, dI = g.dI;
    for (int e = lane; e < dI * HIM; e += 64) {
      const int x = e / HIM, h = e - x * HIM;
      qT[e] = h < HI ? to_f32(qI[((int64_t)t * HI + h) * dI + x]) : 0.0f;
    }
    if (lane < HIM) wsh[lane] = lane < HI ? w[(int64_t)t * HI + lane] : 0.0f;
    __syncthreads();
    if (j0 < nb) {
      float acc[HIM][4];
#pragma unroll
      for (int h = 0; h < HIM; ++h) acc[h][0] = acc[h][1] = acc[h][2] = acc[h][3] = 0.0f;
      const float* pb = pooled + (int64_t)qp.b * dI * g.pooled_ld + j0;
      for (int x = 0; x < dI; ++x) {
        const float4 pk = *reinterpret_cast<const float4*>(pb + (int64_t)x * g.pooled_ld);
#pragma unroll
        for (int h = 0; h < HIM; ++h) {
          const float qv = qT[x * HIM + h];
          acc[h][0] = fmaf(qv, pk.x, acc[h][0]);
          acc[h][1] = fmaf(qv, pk.y, acc[h][1]);
          acc[h][2] = fmaf(qv, pk.z, acc[h][2]);
          acc[h][3] = fmaf(qv, pk.w, acc[h][3]);
        }
      }
#pragma unroll
      for (int h = 0; h < HIM; ++h) {
        if (h < HI) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float a = g.idx_scale * acc[h][i];
            a = (a > 0.0f) ? a : 0.0f;
            s[i] = fmaf(wsh[h], a, s[i]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = j0 + i;
    if (j < g.nbcap) srow[j] = (j < nb) ? s[i] : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Exclusive prefix sum over a 256-thread workgroup (4 waves).
__device__ __forceinline__ int block_excl_scan(int v, int* total, int* sh) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
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

// select: one 256-thread workgroup per query.
__global__ __launch_bounds__(256) void select_kernel(Geo g, const float* __restrict__ scores,
                                                     int32_t* __restrict__ sel,
                                                     int32_t* __restrict__ n_blocks) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix;
  __shared__ int s_want;
  __shared__ int sh[4];
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
  const float* srow = scores + (int64_t)t * g.nbcap;
  uint32_t prefix = 0, mask = 0;
  int want = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int j = tid; j < nb; j += 256) {
      const uint32_t key = score_key(srow[j]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    const int d = 255 - tid;  // thread order = descending digit
    const int c = static_cast<int>(hist[d]);
    int tot;
    const int above = block_excl_scan(c, &tot, sh);  // matching keys with digit > d
    if (above < want && above + c >= want) {
      s_prefix = prefix | (static_cast<uint32_t>(d) << shift);
      s_want = want - above;
    }
    __syncthreads();
    prefix = s_prefix;
    want = s_want;
    mask |= 255u << shift;
  }
  // prefix is the k-th largest key; keep every larger key and the `want`
  // lowest-index keys equal to it, written in ascending block order.
  int base = 0, eq_base = 0;
  for (int c0 = 0; c0 < nb; c0 += 256) {
    const int j = c0 + tid;
    const uint32_t key = j < nb ? score_key(srow[j]) : 0u;
    const int gt = (j < nb) && key > prefix;
    const int eq = (j < nb) && key == prefix;
    int eq_tot, take_tot;
    const int eq_rank = eq_base + block_excl_scan(eq, &eq_tot, sh);
    const int take = gt || (eq && eq_rank < want);
    const int pos = base + block_excl_scan(take, &take_tot, sh);
    if (take && pos < k) out[pos] = j;
    base += take_tot;
    eq_base += eq_tot;
  }
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
  const int i0 = split * plan.split_tokens;
  const int i1 = min(i0 + plan.split_tokens, L.n_list);
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
      P[G * D + G + h] = l[h];
    }
  }
}

template <typename E, int G, int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(Geo g, AttnPlan plan,
                                                           const float* __restrict__ part,
                                                           const E* __restrict__ gate,
                                                           E* __restrict__ out) {
  const int unit = blockIdx.x;
  const int t = unit / g.Hkv, kvh = unit - t * g.Hkv;
  const QueryPos qp = query_pos(g, t);
  if (!qp.ok) return;
  const float* P0 = part + (int64_t)unit * plan.n_splits * (G * (D + 2));
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int h = e / D, d = e - h * D;
    float M = -INFINITY;
    for (int s = 0; s < plan.n_splits; ++s) M = fmaxf(M, P0[s * (G * (D + 2)) + G * D + h]);
    float Lsum = 0.0f, O = 0.0f;
    for (int s = 0; s < plan.n_splits; ++s) {
      const float* P = P0 + s * (G * (D + 2));
      const float ms = P[G * D + h];
      if (ms == -INFINITY) continue;
      const float wgt = exp2f(ms - M);
      Lsum = fmaf(P[G * D + G + h], wgt, Lsum);
      O = fmaf(P[h * D + d], wgt, O);
    }
    const int64_t idx = ((int64_t)t * g.Hq + kvh * G + h) * D + d;
    const float sg = 1.0f / (1.0f + expf(-to_f32(gate[idx])));
    out[idx] = from_f32<E>(Lsum > 0.0f ? O / Lsum * sg : 0.0f);
  }
}

template <typename E, int G, int D>
hipError_t attend_impl(const Geo& g, const AttnPlan& plan, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* sel, const int32_t* n_blocks,
                       const void* gate, void* out, float* part, hipStream_t st) {
  dim3 grid(g.T * g.Hkv, plan.n_splits);
  attn_split_kernel<E, G, D><<<grid, 64, 0, st>>>(
      g, plan, static_cast<const E*>(q), static_cast<const E*>(k_cache),
      static_cast<const E*>(v_cache), sel, n_blocks, static_cast<const E*>(gate),
      static_cast<E*>(out), part);
  if (plan.n_splits > 1) {
    attn_combine_kernel<E, G, D><<<g.T * g.Hkv, 256, 0, st>>>(
        g, plan, part, static_cast<const E*>(gate), static_cast<E*>(out));
  }
  return hipGetLastError();
}

template <typename E, int G>
hipError_t attend_d(const Geo& g, const AttnPlan& plan, const void* q, const void* kc,
                    const void* vc, const int32_t* sel, const int32_t* nb, const void* gate,
                    void* out, float* part, hipStream_t st) {
  if (g.D == 64) return attend_impl<E, G, 64>(g, plan, q, kc, vc, sel, nb, gate, out, part, st);
  return attend_impl<E, G, 128>(g, plan, q, kc, vc, sel, nb, gate, out, part, st);
}

template <typename E>
hipError_t attend_g(const Geo& g, const AttnPlan& plan, const void* q, const void* kc,
                    const void* vc, const int32_t* sel, const int32_t* nb, const void* gate,
                    void* out, float* part, hipStream_t st) {
  switch (g.G) {
    case 1: return attend_d<E, 1>(g, plan, q, kc, vc, sel, nb, gate, out, part, st);
    case 2: return attend_d<E, 2>(g, plan, q, kc, vc, sel, nb, gate, out, part, st);
    case 4: return attend_d<E, 4>(g, plan, q, kc, vc, sel, nb, gate, out, part, st);
    case 8: return attend_d<E, 8>(g, plan, q, kc, vc, sel, nb, gate, out, part, st);
    default: return attend_d<E, 16>(g, plan, q, kc, vc, sel, nb, gate, out, part, st);
  }
}

template <typename E>
hipError_t score_h(const Geo& g, const void* qI, const float* w, const float* pooled,
                   float* scores, hipStream_t st) {
  dim3 grid(g.T, (g.nbcap + 255) / 256);
  if (g.HI <= 4) {
    score_kernel<E, 4><<<grid, 64, 0, st>>>(g, static_cast<const E*>(qI), w, pooled, scores);
  } else if (g.HI <= 8) {
    score_kernel<E, 8><<<grid, 64, 0, st>>>(g, static_cast<const E*>(qI), w, pooled, scores);
  } else {
    score_kernel<E, 16><<<grid, 64, 0, st>>>(g, static_cast<const E*>(qI), w, pooled, scores);
  }
  return hipGetLastError();
}

}  // namespace

bool attend_supported(int G, int D) {
  return (G == 1 || G == 2 || G == 4 || G == 8 || G == 16) && (D == 64 || D == 128);
}

hipError_t launch_append_pool(const Geo& g, int elem, const void* k_new, const void* v_new,
                              const void* kI_new, void* k_cache, void* v_cache, void* kI_cache,
                              float* pooled, hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  if (elem == kBF16) {
    append_pool_kernel<uint16_t><<<g.T, 256, 0, st>>>(
        g, static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
        static_cast<const uint16_t*>(kI_new), static_cast<uint16_t*>(k_cache),
        static_cast<uint16_t*>(v_cache), static_cast<uint16_t*>(kI_cache), pooled);
  } else {
    append_pool_kernel<float><<<g.T, 256, 0, st>>>(
        g, static_cast<const float*>(k_new), static_cast<const float*>(v_new),
        static_cast<const float*>(kI_new), static_cast<float*>(k_cache),
        static_cast<float*>(v_cache), static_cast<float*>(kI_cache), pooled);
  }
  return hipGetLastError();
}

hipError_t launch_score(const Geo& g, int elem, const void* qI, const float* w,
                        const float* pooled, float* scores, hipStream_t st) {
  if (g.T == 0 || g.nbcap == 0) return hipSuccess;
  return elem == kBF16 ? score_h<uint16_t>(g, qI, w, pooled, scores, st)
                       : score_h<float>(g, qI, w, pooled, scores, st);
}

hipError_t launch_select(const Geo& g, const float* scores, int32_t* sel, int32_t* n_blocks,
                         hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  select_kernel<<<g.T, 256, 0, st>>>(g, scores, sel, n_blocks);
  return hipGetLastError();
}

hipError_t launch_attend(const Geo& g, int elem, const AttnPlan& plan, const void* q,
                         const void* k_cache, const void* v_cache, const int32_t* sel,
                         const int32_t* n_blocks, const void* gate, void* out, float* part,
                         hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  return elem == kBF16
             ? attend_g<uint16_t>(g, plan, q, k_cache, v_cache, sel, n_blocks, gate, out, part, st)
             : attend_g<float>(g, plan, q, k_cache, v_cache, sel, n_blocks, gate, out, part, st);
}

}  // namespace qsa
