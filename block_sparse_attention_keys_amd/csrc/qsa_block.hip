// The QSA attention block around the hot path, for gfx950 (MI355X).
//
// The llama.cpp PR #27739 page, LocalAI QSA-block commit (opening paragraph)
// lists the block end to end: q/k/v/o projections, q/k norms with the
// (1 + w) weight polarity, RoPE, the indexer, the gather consumer, the
// sigmoid output gate and o_proj; its fresh-review section has the query
// side and the pooled indexer keys rotated with one set of angles.
//
// Kernels:
//   proj_gemm   C = A . B^T for the projections (A [M][K] activations, B
//               [N][K] Linear weights, both bf16 with K contiguous), on
//               v_mfma_f32_16x16x32_bf16 with both operands loaded straight
//               from memory (their MFMA layouts are 16 contiguous bytes of a
//               row per lane).  A workgroup owns a 32x32 output tile; its four
//               waves take interleaved k-steps of the workgroup's k range and
//               are summed through LDS; the grid splits K further into fp32
//               partials when the tiles alone cannot fill the chip (decode).
//   proj_gemm_tiled  the same product for many rows (prefill): 128 x 128
//               workgroup tiles staged through LDS, double-buffered.  Such
//               products go to hipBLASLt first (qsa_blas.hip, plain library
//               GEMMs); this kernel runs where hipBLASLt cannot.
//   block_prep  per (token, projection row): sums the partials of the
//               stacked input projection, RMSNorm (1 + w) and RoPE on the q
//               and k heads, RoPE on the indexer query heads, bf16 rounding of
//               everything the QSA path reads; head weights all ones.  One
//               row per wave for decode-sized calls, four (loads of all four
//               in flight) for prefill-sized ones; the token's rotary factors
//               once per workgroup.
//   proj_reduce sums the partials of o_proj into the bf16 output.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "qsa_internal.h"

namespace qsa {
namespace {

#include "qsa_device.h"

// ---------------------------------------------------------------------------
// Projection GEMM.  Matrix-core layout of v_mfma_f32_16x16x32_bf16 (l = lane):
//   A[i][k]: i = l%16, k = 8*(l/16) + e;  B[k][j]: j = l%16, k = 8*(l/16) + e;
//   C[i][j]: j = l%16, i = 4*(l/16) + r.
// A lane's A fragment is 16 bytes of activation row (m0 + l%16) at column
// k0 + 8*(l/16); its B fragment 16 bytes of weight row (n0 + l%16) there too.
constexpr int kGemmSteps = 8;  // k-steps (32 wide) a wave requests at once
// Offset of a row past the matrix: every offset from here on is past the end
// (the host keeps both operands under 2 GiB), also after adding a k offset.
constexpr uint32_t kGemmOob = 0x80000000u;

__global__ __launch_bounds__(256) void proj_gemm_kernel(const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ B,
                                                        float* __restrict__ part,
                                                        uint16_t* __restrict__ out, int M, int N,
                                                        int K, int k_split) {
  __shared__ float red[4][32][33];
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c16 = lane & 15, q4 = lane >> 4;
  const int n0 = blockIdx.x * 32, m0 = blockIdx.y * 32, s = blockIdx.z;
  const int kb = s * k_split, ke = min(K, kb + k_split);
  const int nsteps = (ke - kb) >> 5;  // k_split and K are multiples of 32
  const __amdgpu_buffer_rsrc_t ars = buffer_rsrc(A, (uint32_t)((int64_t)M * K * 2));
  const __amdgpu_buffer_rsrc_t brs = buffer_rsrc(B, (uint32_t)((int64_t)N * K * 2));
  // Row offsets (bytes) of this lane's two A rows and two B rows; rows past
  // the matrix read past the end of the buffer and come back zero.
  uint32_t aoff[2], boff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + 16 * i + c16, n = n0 + 16 * i + c16;
    aoff[i] = m < M ? (uint32_t)(m * K + 8 * q4) * 2u : kGemmOob;
    boff[i] = n < N ? (uint32_t)(n * K + 8 * q4) * 2u : kGemmOob;
  }
  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // Wave wid takes k-steps wid, wid + 4, wid + 8, ... of [kb, ke).
  for (int st0 = wid; st0 < nsteps; st0 += 4 * kGemmSteps) {
    uint4 af[kGemmSteps][2], bfr[kGemmSteps][2];
#pragma unroll
    for (int u = 0; u < kGemmSteps; ++u) {
      const int stp = st0 + 4 * u;
      const uint32_t kbyte = (uint32_t)(kb + 32 * stp) * 2u;
      const bool live = stp < nsteps;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[u][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 ars, live ? aoff[i] + kbyte : kGemmOob, 0, 0));
        bfr[u][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  brs, live ? boff[i] + kbyte : kGemmOob, 0, 0));
      }
    }
    // All of this round's loads are in flight before the first MFMA.  (Steps
    // past the range loaded zeros: their products add nothing.)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kGemmSteps; ++u) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, af[u][i]), __builtin_bit_cast(bf16x8_t, bfr[u][j]),
              acc[i][j], 0, 0, 0);
    }
  }
  // C fragment: row 16 i + 4 q4 + r, column 16 j + c16.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wid][16 * i + 4 * q4 + r][16 * j + c16] = acc[i][j][r];
  __syncthreads();
  // Sum the four waves (in wave order) and store this split's partial tile,
  // or (out given: one split) the bf16 result.
  float* P = part + (int64_t)s * M * N;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int idx = threadIdx.x + 256 * e, rr = idx >> 5, cc = idx & 31;
    const int m = m0 + rr, n = n0 + cc;
    const float v = ((red[0][rr][cc] + red[1][rr][cc]) + red[2][rr][cc]) + red[3][rr][cc];
    if (m < M && n < N) {
      if (out != nullptr) out[(int64_t)m * N + n] = bf16_rne(v);
      else P[(int64_t)m * N + n] = v;
    }
  }
}

// The product for many rows (prefill): a workgroup computes a 128 x 128 tile
// through LDS.  Per k-step of 32, the 256 threads bring the A and B tiles
// (128 rows x 64 bytes each, 16 bytes per thread and load, two loads each)
// into LDS rows padded to 40 elements (80 bytes: the 16 rows a fragment read
// touches fall on distinct banks), double-buffered, the next step's loads in
// flight while the current step multiplies.  Wave (wm, wn) owns the 64 x 64
// quarter at rows 64 wm, columns 64 wn: per k-step 4 A and 4 B fragments
// from LDS and 16 MFMAs.
constexpr int kTile = 128, kLdsRow = 40;

__global__ __launch_bounds__(256) void proj_gemm_tiled_kernel(const uint16_t* __restrict__ A,
                                                              const uint16_t* __restrict__ B,
                                                              float* __restrict__ part,
                                                              uint16_t* __restrict__ out, int M,
                                                              int N, int K) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kTile * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kTile * kLdsRow];
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, q4 = lane >> 4, wm = wid >> 1, wn = wid & 1;
  const int m0 = blockIdx.y * kTile, n0 = blockIdx.x * kTile;
  const __amdgpu_buffer_rsrc_t ars = buffer_rsrc(A, (uint32_t)((int64_t)M * K * 2));
  const __amdgpu_buffer_rsrc_t brs = buffer_rsrc(B, (uint32_t)((int64_t)N * K * 2));
  // This thread's two 16-byte pieces of each tile: rows tid/4 and tid/4 + 64,
  // bytes 16 (tid % 4) of the row's 64-byte k-step.
  const int lr = tid >> 2, lc = tid & 3;
  uint32_t aoff[2], boff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int m = m0 + lr + 64 * h, n = n0 + lr + 64 * h;
    aoff[h] = m < M ? (uint32_t)(m * K + 8 * lc) * 2u : kGemmOob;
    boff[h] = n < N ? (uint32_t)(n * K + 8 * lc) * 2u : kGemmOob;
  }
  uint4 ga[2], gb[2];
  auto fetch = [&](int kt) {
    const uint32_t kbyte = (uint32_t)kt * 64u;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ga[h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ars, aoff[h] + kbyte, 0, 0));
      gb[h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(brs, boff[h] + kbyte, 0, 0));
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<uint4*>(&As[buf][(lr + 64 * h) * kLdsRow + 8 * lc]) = ga[h];
      *reinterpret_cast<uint4*>(&Bs[buf][(lr + 64 * h) * kLdsRow + 8 * lc]) = gb[h];
    }
  };
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int KT = K >> 5;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) fetch(kt + 1);
    uint4 af[4], bfr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      af[i] = *reinterpret_cast<const uint4*>(&As[buf][(64 * wm + 16 * i + c16) * kLdsRow + 8 * q4]);
      bfr[i] = *reinterpret_cast<const uint4*>(&Bs[buf][(64 * wn + 16 * i + c16) * kLdsRow + 8 * q4]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[i]),
                                                            __builtin_bit_cast(bf16x8_t, bfr[j]),
                                                            acc[i][j], 0, 0, 0);
    if (kt + 1 < KT) stash(buf ^ 1);
    __syncthreads();
  }
  // C fragment: row 16 i + 4 q4 + r, column 16 j + c16 of the wave's quarter.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 64 * wm + 16 * i + 4 * q4 + r, n = n0 + 64 * wn + 16 * j + c16;
        if (m < M && n < N) {
          if (out != nullptr) out[(int64_t)m * N + n] = bf16_rne(acc[i][j][r]);
          else part[(int64_t)m * N + n] = acc[i][j][r];
        }
      }
}

// Sum of the S (<= kMaxSplits) partials of element idx, splits in order; the
// S loads are all issued before the first add (S is the same for the whole
// grid, so the guards skip the loads of absent splits without diverging).
constexpr int kMaxSplits = 16;
__device__ __forceinline__ float sum_parts(const float* part, int S, int64_t MN, int64_t idx) {
  if (S == 1) return part[idx];
  float p[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) p[s] = s < S ? part[s * MN + idx] : 0.0f;
  float v = 0.0f;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    if (s < S) v += p[s];
  return v;
}

__global__ __launch_bounds__(256) void proj_reduce_kernel(const float* __restrict__ part, int S,
                                                          int64_t MN,
                                                          uint16_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < MN) out[idx] = bf16_rne(sum_parts(part, S, MN, idx));
}

struct QueryPosB {
  int p;
  bool ok;
};
// Position of new token t (cu_q / past_len, as the rest of the path).
__device__ QueryPosB token_pos(const Geo& g, int t) {
  int lo = 0, hi = g.B - 1;
  while (lo < hi) {  // last b with cu_q[b] <= t
    const int mid = (lo + hi + 1) >> 1;
    if (g.cu_q[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  const int b = lo, p = g.past_len[b] + (t - g.cu_q[b]);
  return {p, p >= 0 && p < g.cap};
}

// Grid (token, group of 4 RPW rows); each wave takes RPW consecutive rows of
// the stacked input projection (q heads, gate heads, k heads, v heads,
// indexer-query heads, the indexer key), requests the partial sums of all of
// them before it uses the first, then finishes them one by one.  Lane l
// holds values l and l + 64 of a row.
struct PrepRow {
  int kind, head, base, len;  // kind: 0 q, 1 gate, 2 k, 3 v, 4 indexer q, 5 indexer k
};
__device__ __forceinline__ PrepRow prep_row(const Geo& g, int rw) {
  const int D = g.D, Hq = g.Hq, Hkv = g.Hkv, HI = g.HI, dI = g.dI;
  if (rw < Hq) return {0, rw, rw * D, D};
  if (rw < 2 * Hq) return {1, rw - Hq, rw * D, D};
  if (rw < 2 * Hq + Hkv) return {2, rw - 2 * Hq, rw * D, D};
  if (rw < 2 * Hq + 2 * Hkv) return {3, rw - 2 * Hq - Hkv, rw * D, D};
  if (rw < 2 * Hq + 2 * Hkv + HI) {
    const int head = rw - 2 * Hq - 2 * Hkv;
    return {4, head, (2 * Hq + 2 * Hkv) * D + head * dI, dI};
  }
  return {5, 0, (2 * Hq + 2 * Hkv) * D + HI * dI, dI};
}

// Rotate-half at value x of a row with the token's factors c[i] = cos(pos f_i),
// s[i] = sin(pos f_i) (computed in fp64, rounded to fp32).
__device__ __forceinline__ float rope_tab(const float* row, int x, int R, const float* c,
                                          const float* s) {
  if (x >= R) return row[x];
  const int h = R >> 1, i = x < h ? x : x - h;
  if (x < h) return row[x] * c[i] - row[x + h] * s[i];
  return row[x] * c[i] + row[i] * s[i];
}

template <int RPW, bool ONE_SPLIT>  // ONE_SPLIT: a.S == 1 (loads need no split sums)
__global__ __launch_bounds__(256) void block_prep_kernel(Geo g, BlockPrepArgs a) {
  __shared__ float rowbuf[4][128];
  __shared__ float cos_tab[2][64], sin_tab[2][64];  // [q/k, indexer q][frequency]
  const int t = blockIdx.x, wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (g.r > 0 && blockIdx.y == 0 && threadIdx.x < g.HI) a.w[(int64_t)t * g.HI + threadIdx.x] = 1.0f;
  const QueryPosB qp = token_pos(g, t);
  const int64_t pos = qp.ok ? qp.p : 0;
  const int D = g.D, Hq = g.Hq, Hkv = g.Hkv, HI = g.HI, dI = g.dI;
  const int n_rows = 2 * Hq + 2 * Hkv + (g.r > 0 ? HI + 1 : 0);
  const int64_t MN = (int64_t)g.T * a.n_in;
  const float* P = a.part + (int64_t)t * a.n_in;
  float* row = rowbuf[wid];
  const int rw0 = (blockIdx.y * 4 + wid) * RPW;
  // requested first (loads complete in order): this thread's rotary
  // frequency and the two norm weights' values of lanes l and l + 64
  // (the table only where the workgroup holds a q, k or indexer-q row)
  const int wg_lo = blockIdx.y * 4 * RPW, wg_hi = min(n_rows, wg_lo + 4 * RPW);
  const auto overlaps = [&](int lo, int hi) { return wg_lo < hi && lo < wg_hi; };
  const bool need_tab = overlaps(0, Hq) || overlaps(2 * Hq, 2 * Hq + Hkv) ||
                        (g.r > 0 && overlaps(2 * Hq + 2 * Hkv, 2 * Hq + 2 * Hkv + HI));
  const int tab_which = threadIdx.x >> 6, tab_i = threadIdx.x & 63;
  const int tab_R = tab_which ? g.idx_rope_dim : a.rotary_dim;
  const bool tab_on = need_tab && threadIdx.x < 128 && tab_i < (tab_R >> 1);
  const double tab_f = tab_on ? (tab_which ? a.idx_freq[tab_i] : a.freq[tab_i]) : 0.0;
  float qn[2], kn[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int x = min(lane + 64 * e, D - 1);
    qn[e] = to_f32(a.q_norm[x]);
    kn[e] = to_f32(a.k_norm[x]);
  }
  float v[RPW][2];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const PrepRow pr = prep_row(g, rw0 + i);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int x = lane + 64 * e;
      const bool ok = rw0 + i < n_rows && x < pr.len;
      if constexpr (ONE_SPLIT) {
        // unconditional loads (at value 0 of the token for absent ones), so
        // all of them are in flight together
        const float val = P[ok ? pr.base + x : 0];
        v[i][e] = ok ? val : 0.0f;
      } else {
        v[i][e] = ok ? sum_parts(P, a.S, MN, pr.base + x) : 0.0f;
      }
    }
  }
  // the token's rotary factors, once per workgroup (every rotated row of the
  // token uses the same 2 x 32 angles), computed while the loads are in flight
  if (need_tab) {  // uniform over the workgroup
    if (tab_on) {
      double sn, cs;
      sincos((double)pos * tab_f, &sn, &cs);
      cos_tab[tab_which][tab_i] = (float)cs;
      sin_tab[tab_which][tab_i] = (float)sn;
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    if (rw0 + i >= n_rows) break;
    const PrepRow pr = prep_row(g, rw0 + i);
    const int kind = pr.kind, head = pr.head, len = pr.len;
    float* vr = v[i];
    if (kind == 0 || kind == 2) {
      // RMSNorm over the head, weight (1 + w).
      const float ss = wave_sum(vr[0] * vr[0] + vr[1] * vr[1]);
      const float inv = 1.0f / sqrtf(ss / (float)len + a.eps);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int x = lane + 64 * e;
        if (x < len) vr[e] = (vr[e] * inv) * (1.0f + (kind == 0 ? qn[e] : kn[e]));
      }
    }
    if (kind == 0 || kind == 2 || kind == 4) {
      const int R = kind == 4 ? g.idx_rope_dim : a.rotary_dim;
      if (R > 0) {
        wave_sync();  // the previous row's reads of the buffer are done
#pragma unroll
        for (int e = 0; e < 2; ++e)
          if (lane + 64 * e < len) row[lane + 64 * e] = vr[e];
        wave_sync();
        float rv[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int x = lane + 64 * e;
          const int which = kind == 4 ? 1 : 0;
          rv[e] = x >= len ? 0.0f : rope_tab(row, x, R, cos_tab[which], sin_tab[which]);
        }
        vr[0] = rv[0];
        vr[1] = rv[1];
      }
    }
    uint16_t* dst;
    switch (kind) {
      case 0: dst = a.q + ((int64_t)t * Hq + head) * D; break;
      case 1: dst = a.gate + ((int64_t)t * Hq + head) * D; break;
      case 2: dst = a.k + ((int64_t)t * Hkv + head) * D; break;
      case 3: dst = a.v + ((int64_t)t * Hkv + head) * D; break;
      case 4: dst = a.q_idx + ((int64_t)t * HI + head) * dI; break;
      default: dst = a.k_idx + (int64_t)t * dI; break;
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int x = lane + 64 * e;
      if (x < len) dst[x] = bf16_rne(vr[e]);
    }
  }
}

}  // namespace

// Many rows (and enough 128 x 128 tiles to fill the chip): the LDS-tiled kernel.
static bool gemm_tiled(int M, int N) {
  return M >= 256 && (int64_t)((M + kTile - 1) / kTile) * ((N + kTile - 1) / kTile) >= 256;
}

int gemm_splits(int M, int N, int K) {
  if (gemm_tiled(M, N)) return 1;
  const int64_t tiles = (int64_t)((M + 31) / 32) * ((N + 31) / 32);
  int64_t S = (384 + tiles - 1) / tiles;
  S = std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(S, K / 128), kMaxSplits));
  const int64_t ks = ((K + S - 1) / S + 127) / 128 * 128;
  return (int)((K + ks - 1) / ks);
}

int gemm_k_split(int K, int S) { return (int)(((K + S - 1) / S + 127) / 128 * 128); }

hipError_t launch_proj_gemm(const void* A, const void* B, float* part, void* out_bf16, int M,
                            int N, int K, int S, hipStream_t st) {
  const int ks = gemm_k_split(K, S);
  uint16_t* out = S == 1 ? static_cast<uint16_t*>(out_bf16) : nullptr;
  if (gemm_tiled(M, N) && S == 1) {
    // a plain GEMM: hipBLASLt's tuned kernels where they run, else our own
    const hipError_t e = lt_gemm(A, B, out != nullptr ? static_cast<void*>(out)
                                                       : static_cast<void*>(part),
                                 out == nullptr, M, N, K, st);
    if (e != hipErrorNotSupported) return e;
    dim3 grid((N + kTile - 1) / kTile, (M + kTile - 1) / kTile);
    proj_gemm_tiled_kernel<<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(A),
                                                 static_cast<const uint16_t*>(B), part, out, M, N,
                                                 K);
    return hipGetLastError();
  }
  dim3 grid((N + 31) / 32, (M + 31) / 32, S);
  proj_gemm_kernel<<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(A),
                                         static_cast<const uint16_t*>(B), part, out, M, N, K, ks);
  return hipGetLastError();
}

hipError_t launch_proj_reduce(const float* part, int S, int64_t MN, void* out, hipStream_t st) {
  proj_reduce_kernel<<<(unsigned)((MN + 255) / 256), 256, 0, st>>>(part, S, MN,
                                                                   static_cast<uint16_t*>(out));
  return hipGetLastError();
}

hipError_t launch_block_prep(const Geo& g, const BlockPrepArgs& a, hipStream_t st) {
  const int n_rows = 2 * g.Hq + 2 * g.Hkv + (g.r > 0 ? g.HI + 1 : 0);
  // prefill-sized calls: 4 rows per wave (loads of all four in flight);
  // decode-sized ones keep one row per wave and more workgroups
  if (g.T >= 512 && a.S == 1)
    block_prep_kernel<4, true><<<dim3(g.T, (n_rows + 15) / 16), 256, 0, st>>>(g, a);
  else block_prep_kernel<1, false><<<dim3(g.T, (n_rows + 3) / 4), 256, 0, st>>>(g, a);
  return hipGetLastError();
}

}  // namespace qsa
