// Key-stationary prefill attention for gfx950 (bf16, D = 128).
//
// In a prefill chunk every query picks its own k blocks (plus its tail), but
// all of them pick from the same few hundred candidate blocks, so each block
// is picked by hundreds of the chunk's queries.  A per-query kernel gathers
// every picked block once per query (8 flop per byte gathered); this path
// turns the selection around instead:
//
//   ks_count, ks_scan, ks_scatter   the plan: per sequence, a counting sort
//              of the (query, slot) entries of the selection (and each
//              query's tail) by block: the block's list of queries, cut into
//              work items of up to kKsItemMax queries.  Where a sequence has
//              at most kScanThreads candidate blocks, ks_scan_scatter does
//              the last two steps in one launch.
//   ks_attn    one workgroup per (item, KV head): the block's K and V rows go
//              to LDS once; the item's queries run through it 64 (query,
//              head) rows at a time as dense bf16 MFMA tiles, S^T = K Q^T
//              then O^T = V^T P^T, with a causal mask per row (the tail block
//              of a query is partial).  Each row's partial state is stored:
//              its output normalised by its own sum (bf16; whole 128-byte
//              lines, through an LDS exchange inside the wave) and its base-2
//              log-sum-exp (fp32), at (query, slot, head).
//   ks_merge   per (query, 16 heads), the log-sum-exp merge of the query's
//              slots (its selected blocks, then the tail), then the sigmoid
//              gate (and, for 8-bit caches in the rotated basis, the inverse
//              rotation and the V scale).
//   ks_rotate_q  8-bit caches in the rotated basis: each query row rotated
//              once per sub-batch, for the attention's query operand.
// Calls with more than kKsSubTokens new tokens run in sub-batches of that
// many queries (the partial states of one sub-batch at a time).
//
// The attention is the one of the pages' QSA description (MTPLX "Native
// Backend Components", section "Qwen Sparse Attention": standard gated GQA
// over the per-query selection intersected with the causal mask); the merge
// is the online-softmax state combination that "Porting Qwen4 to llama.cpp",
// section "CUDA Optimization Should Follow State Correctness", names for the
// direct indexed consumer.  Results do not depend on how queries are grouped
// into tiles: every output row of a matrix-core product depends on its own
// row only.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "qsa_internal.h"

namespace qsa {
namespace {

#include "qsa_device.h"

#ifdef QSA_COUNT_KEYS
// Debug builds: (query, K/V row) pairs attended, per KV head.
__device__ unsigned long long g_ks_keys_visited;
#endif

// Two fp32 values -> a bf16 pair (low, high), round to nearest even by the
// hardware conversion.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

constexpr int kRows = 64;    // (query, head) rows per tile of ks_attn (4 waves x 16)
constexpr int kGroup = 64;   // queries per counting group of the plan
constexpr int kRangeGroups = 16;  // groups per query range of the work-item order
constexpr int kScanThreads = 1024;
// Query ranges per sequence in one sub-batch (the scan keeps a register per
// range and block).
constexpr int kMaxRanges = kKsSubTokens / (kGroup * kRangeGroups);
static_assert(kMaxRanges * kGroup * kRangeGroups == kKsSubTokens, "sub-batch cut into whole ranges");

// Entries of a block's query list: the query's index in the call and its slot
// (position in its selection, or k for the tail), packed as t << 12 | slot.
__device__ __forceinline__ uint32_t pack_entry(int t, int slot) {
  return ((uint32_t)t << kKsSlotBits) | (uint32_t)slot;
}

// Sequence b's queries inside this sub-batch [t_lo, t_hi).
struct SeqRange {
  int t0, t1;  // global token indices, t0 <= t1
};
__device__ __forceinline__ SeqRange seq_range(const Geo& g, const KsArgs& a, int b) {
  SeqRange s;
  s.t0 = min(max(g.cu_q[b], a.t_lo), a.t_hi);
  s.t1 = min(max(g.cu_q[b + 1], a.t_lo), a.t_hi);
  return s;
}
// First work item of sequence b's region (the host sizes the item table with
// the same bound: ks_item_bound).
__device__ __forceinline__ int item_base(const KsArgs& a, int b, int t_rel) {
  return (int)(((int64_t)t_rel * a.k1) / a.item_tokens) + b * (a.nr * a.nb1 + 1);
}

// Block of entry (query t at position p = past + t - cu0, slot): the
// selection entry (slots below the query's n_blocks), or the query's tail
// block (slot k, when the tail is not empty); -1 when there is none.
__device__ __forceinline__ int entry_block(const Geo& g, const KsArgs& a,
                                           const int32_t* __restrict__ sel,
                                           const int32_t* __restrict__ nblk, int p, int t,
                                           int slot) {
  if (p < 0 || p >= g.cap) return -1;
  const int n = p + 1, nb = n >> g.log2r;
  if (slot == g.k) return (n > (nb << g.log2r) && nb < a.nb1) ? nb : -1;
  const int nk = max(0, min(nblk[t], min(g.k, nb)));
  if (slot >= nk) return -1;
  const int j = sel[(int64_t)t * g.k + slot];
  return (j >= 0 && j < nb && j < a.nb1) ? j : -1;
}

// Plan, step 1: grid (query group, sequence).  Entries per block of the
// group's kGroup queries, counted in LDS and stored as the group's row of
// the histogram.
__global__ __launch_bounds__(256) void ks_count_kernel(Geo g, KsArgs a,
                                                      const int32_t* __restrict__ sel,
                                                      const int32_t* __restrict__ nblk) {
  extern __shared__ int32_t hist_lds[];
  const int gi = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const SeqRange sr = seq_range(g, a, b);
  const int ta = min(sr.t0 + gi * kGroup, sr.t1), tb = min(sr.t1, ta + kGroup);
  const int past = g.past_len[b], cu0 = g.cu_q[b], K1 = a.k1;
  for (int i = tid; i < a.nb1; i += 256) hist_lds[i] = 0;
  __syncthreads();
  for (int e = tid; e < (tb - ta) * K1; e += 256) {
    const int t = ta + e / K1, slot = e - (e / K1) * K1;
    const int j = entry_block(g, a, sel, nblk, past + (t - cu0), t, slot);
    if (j >= 0) atomicAdd(&hist_lds[j], 1);
  }
  __syncthreads();
  int32_t* row = a.hist + ((int64_t)b * a.ng + gi) * a.nb1;
  for (int i = tid; i < a.nb1; i += 256) row[i] = hist_lds[i];
}

// Block-wide exclusive scan of one int per thread (kScanThreads threads).
__device__ __forceinline__ int scan_excl(int v, int* total, int* sh) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) sh[wid] = x;
  __syncthreads();
  if (wid == 0) {
    int w = lane < kScanThreads / 64 ? sh[lane] : 0;
#pragma unroll
    for (int d = 1; d < kScanThreads / 64; d <<= 1) {
      const int y = __shfl_up(w, d, 64);
      if (lane >= d) w += y;
    }
    if (lane < kScanThreads / 64) sh[lane] = w;  // inclusive wave totals
  }
  __syncthreads();
  const int before = wid > 0 ? sh[wid - 1] : 0;
  *total = sh[kScanThreads / 64 - 1];
  __syncthreads();  // sh is reused by the next scan
  return before + x - v;
}

// Plan, step 2: one workgroup per sequence.  Per block: the total over the
// groups and the block's first list position (blocks ascending; inside a
// block, groups in order).  Work items are cut per (query range of
// kRangeGroups groups, block), ranges outermost: items dispatched together
// then read the queries of one range, which stay in the L2 of their XCD.
// Unused item slots of the sequence's region are written empty.  The
// histogram is read once, 32 or 64 loads per thread in flight at a time, and its
// per-range sums stay in registers for both scans.
template <int PER>  // consecutive blocks per thread (PER * kScanThreads >= nb1)
__global__ __launch_bounds__(kScanThreads) void ks_scan_kernel(Geo g, KsArgs a) {
  __shared__ int sh[kScanThreads / 64];
  const int b = blockIdx.x, tid = threadIdx.x;
  const SeqRange sr = seq_range(g, a, b);
  const int NB1 = a.nb1, ng = a.ng;
  int32_t* rows = a.hist + (int64_t)b * ng * NB1;
  const int j0 = tid * PER;
  // c[r][i]: entries of block j0 + i from the groups of range r.  Each row
  // of the histogram is replaced by the entries of the block from the groups
  // before it (the scatter's offset inside the block's list).
  int c[kMaxRanges][PER], run[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    run[i] = 0;
#pragma unroll
    for (int r = 0; r < kMaxRanges; ++r) c[r][i] = 0;
  }
  if (j0 < NB1) {
    constexpr int GB = (PER == 1 ? 64 : 32) / PER;  // group rows per batch
#pragma unroll
    for (int g0 = 0; g0 < kMaxRanges * kRangeGroups; g0 += GB) {
      if (g0 >= ng) break;
      int v[GB][PER];
#pragma unroll
      for (int x = 0; x < GB; ++x)
#pragma unroll
        for (int i = 0; i < PER; ++i)
          v[x][i] = (g0 + x < ng && j0 + i < NB1) ? rows[(int64_t)(g0 + x) * NB1 + j0 + i] : 0;
#pragma unroll
      for (int x = 0; x < GB; ++x)
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          if (g0 + x < ng && j0 + i < NB1) rows[(int64_t)(g0 + x) * NB1 + j0 + i] = run[i];
          run[i] += v[x][i];
          c[(g0 + x) / kRangeGroups][i] += v[x][i];
        }
    }
  }
  const int n_ranges = (ng + kRangeGroups - 1) / kRangeGroups;
  int tot[PER], ents = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    tot[i] = 0;
#pragma unroll
    for (int r = 0; r < kMaxRanges; ++r) tot[i] += c[r][i];
    ents += tot[i];
  }
  int total_ents;
  const int ent_before = scan_excl(ents, &total_ents, sh);
  const int list0 = (sr.t0 - a.t_lo) * a.k1;  // the sequence's list region
  int32_t* boff = a.boff + (int64_t)b * NB1;
  int pos[PER];  // list position of each block's next range
  {
    int o = list0 + ent_before;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (j0 + i < NB1) boff[j0 + i] = o;
      pos[i] = o;
      o += tot[i];
    }
  }
  const int base = item_base(a, b, sr.t0 - a.t_lo);
  const int base_next = item_base(a, b + 1, sr.t1 - a.t_lo);
  int it0 = base;
#pragma unroll
  for (int r = 0; r < kMaxRanges; ++r) {
    if (r >= n_ranges) break;  // uniform: every thread reaches the same scans
    int items = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) items += (c[r][i] + a.item_tokens - 1) / a.item_tokens;
    int total_items;
    int it = it0 + scan_excl(items, &total_items, sh);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      for (int x = 0; x < c[r][i]; x += a.item_tokens, ++it)
        a.items[it] = make_int4(pos[i] + x, j0 + i, min(a.item_tokens, c[r][i] - x), b);
      pos[i] += c[r][i];
    }
    it0 += total_items;
  }
  for (int x = it0 + tid; x < base_next; x += kScanThreads) a.items[x] = make_int4(0, 0, 0, b);
}

// Plan, step 3: grid (query group, sequence).  Each entry goes to its
// block's list at the block's first position, plus the entries of the
// block from earlier groups (the scan left them in the group's histogram
// row), plus its rank among this group's entries of the block.
__global__ __launch_bounds__(256) void ks_scatter_kernel(Geo g, KsArgs a,
                                                        const int32_t* __restrict__ sel,
                                                        const int32_t* __restrict__ nblk) {
  extern __shared__ int32_t pos_lds[];
  const int gi = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const SeqRange sr = seq_range(g, a, b);
  const int ta = min(sr.t0 + gi * kGroup, sr.t1), tb = min(sr.t1, ta + kGroup);
  if (ta >= tb) return;
  const int past = g.past_len[b], cu0 = g.cu_q[b], K1 = a.k1, NB1 = a.nb1;
  const int32_t* before = a.hist + ((int64_t)b * a.ng + gi) * NB1;
  const int32_t* boff = a.boff + (int64_t)b * NB1;
  for (int j = tid; j < NB1; j += 256) pos_lds[j] = boff[j] + before[j];
  __syncthreads();
  for (int e = tid; e < (tb - ta) * K1; e += 256) {
    const int t = ta + e / K1, slot = e - (e / K1) * K1;
    const int j = entry_block(g, a, sel, nblk, past + (t - cu0), t, slot);
    if (j >= 0) a.list[atomicAdd(&pos_lds[j], 1)] = pack_entry(t, slot);
  }
}

// Plan, steps 2 and 3 in one launch, for sequences of at most kScanThreads
// candidate blocks (+ the tail): grid (query group, sequence), one thread per
// block.  Each workgroup reads its sequence's whole histogram (each thread
// its block's column, one entry per group) and derives its own list
// positions from it: the block's first position from the sums of every group, then the
// entries of the block from the groups before this one.  The group-0
// workgroup also cuts the work items, in the same order and form as
// ks_scan_kernel.  Without the one-workgroup scan between them, counting and
// scattering are two launches instead of three.
__global__ __launch_bounds__(kScanThreads) void ks_scan_scatter_kernel(
    Geo g, KsArgs a, const int32_t* __restrict__ sel, const int32_t* __restrict__ nblk) {
  extern __shared__ int32_t pos_lds[];
  __shared__ int sh[kScanThreads / 64];
  const int gi = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const SeqRange sr = seq_range(g, a, b);
  const int ta = min(sr.t0 + gi * kGroup, sr.t1), tb = min(sr.t1, ta + kGroup);
  if (gi > 0 && ta >= tb) return;  // (the whole workgroup: no queries in this group)
  const int NB1 = a.nb1, ng = a.ng, j = tid;
  const int32_t* rows = a.hist + (int64_t)b * ng * NB1;
  // c[r]: entries of block j from the groups of range r; before: from the
  // groups ahead of this one
  int c[kMaxRanges], before = 0;
#pragma unroll
  for (int r = 0; r < kMaxRanges; ++r) c[r] = 0;
  if (j < NB1) {
    constexpr int GB = 32;  // group rows per batch of loads
#pragma unroll
    for (int g0 = 0; g0 < kMaxRanges * kRangeGroups; g0 += GB) {
      if (g0 >= ng) break;
      int v[GB];
#pragma unroll
      for (int x = 0; x < GB; ++x) v[x] = (g0 + x < ng) ? rows[(int64_t)(g0 + x) * NB1 + j] : 0;
#pragma unroll
      for (int x = 0; x < GB; ++x) {
        c[(g0 + x) / kRangeGroups] += v[x];
        before += (g0 + x < gi) ? v[x] : 0;
      }
    }
  }
  int tot = 0;
#pragma unroll
  for (int r = 0; r < kMaxRanges; ++r) tot += c[r];
  int total_ents;
  const int ent_before = scan_excl(tot, &total_ents, sh);
  const int o = (sr.t0 - a.t_lo) * a.k1 + ent_before;  // block j's first list position
  if (j < NB1) pos_lds[j] = o + before;
  if (gi == 0) {
    const int n_ranges = (ng + kRangeGroups - 1) / kRangeGroups;
    const int base_next = item_base(a, b + 1, sr.t1 - a.t_lo);
    int it0 = item_base(a, b, sr.t0 - a.t_lo), pos = o;
#pragma unroll
    for (int r = 0; r < kMaxRanges; ++r) {
      if (r >= n_ranges) break;  // uniform: every thread reaches the same scans
      int total_items;
      int it = it0 + scan_excl((c[r] + a.item_tokens - 1) / a.item_tokens, &total_items, sh);
      for (int x = 0; x < c[r]; x += a.item_tokens, ++it)
        a.items[it] = make_int4(pos + x, j, min(a.item_tokens, c[r] - x), b);
      pos += c[r];
      it0 += total_items;
    }
    for (int x = it0 + tid; x < base_next; x += kScanThreads) a.items[x] = make_int4(0, 0, 0, b);
    if (ta >= tb) return;  // (the whole workgroup: a sequence without queries here)
  }
  __syncthreads();
  const int past = g.past_len[b], cu0 = g.cu_q[b], K1 = a.k1;
  for (int e = tid; e < (tb - ta) * K1; e += kScanThreads) {
    const int t = ta + e / K1, slot = e - (e / K1) * K1;
    const int jj = entry_block(g, a, sel, nblk, past + (t - cu0), t, slot);
    if (jj >= 0) a.list[atomicAdd(&pos_lds[jj], 1)] = pack_entry(t, slot);
  }
}

// 8-bit K/V in the rotated basis: each query row of the sub-batch rotated
// once (q' = H q, the Sylvester Hadamard matrix in the standard butterfly
// order: dim bit 0 first) and rounded to bf16 for the matrix cores, as the
// decode kernel does with its staged query.  16 lanes per (query, head) row,
// 4 rows per wave: lane l16 holds dims 8 l16 .. +7 (16-byte loads and
// stores), bits 0-2 of the dim in the lane, bits 3-6 across lanes.
__global__ __launch_bounds__(256) void ks_rotate_q_kernel(Geo g, KsArgs a,
                                                         const uint16_t* __restrict__ q) {
  const int lane = threadIdx.x & 63, l16 = lane & 15;
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);  // (t - t_lo) * Hq + h
  const bool ok = row < (int64_t)(a.t_hi - a.t_lo) * g.Hq;
  const uint4 pr =
      ok ? *reinterpret_cast<const uint4*>(q + ((int64_t)a.t_lo * g.Hq + row) * 128 + 8 * l16)
         : make_uint4(0u, 0u, 0u, 0u);
  const uint32_t pw[4] = {pr.x, pr.y, pr.z, pr.w};
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf_lo(pw[i]);
    v[2 * i + 1] = bf_hi(pw[i]);
  }
#pragma unroll
  for (int len = 1; len < 8; len <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (!(i & len)) {
        const float x = v[i], y = v[i + len];
        v[i] = x + y;
        v[i + len] = x - y;
      }
#pragma unroll
  for (int dl = 1; dl < 16; dl <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = fwht_cross(v[i], dl, (l16 & dl) != 0);
  if (ok)
    *reinterpret_cast<uint4*>(a.qrot + row * 128 + 8 * l16) =
        make_uint4(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]),
                   pack_bf16(v[6], v[7]));
}

// One workgroup (4 waves) per (work item, KV head).  Matrix-core layout of
// v_mfma_f32_16x16x32_bf16 (l = lane, c16 = l % 16, grp = l / 16):
//   A[i][k]: i = c16, k = 8 grp + e;  B[k][j]: j = c16, k = 8 grp + e;
//   C[i][j]: j = c16, i = 4 grp + r.
// The item's queries run through the block 64 (query, head) rows at a
// time; wave w holds rows 16 w .. 16 w + 15 of each tile (row R = query R / G
// of the tile, head R % G), lane c16 row 16 w + c16.
//   S^T[key][row] = K (A: key 16 n + c16 from LDS, 272-byte rows) x Q^T
//     (B: the row's query, 16 bytes from memory, the next tile's requested
//     during this one): a lane holds row c16's scores of keys 16 n + 4 grp + r;
//   the row's softmax over the block's keys it may see (causal mask), in
//     base 2: in-lane over 4 KT keys, then two row swaps; p / l rounded to
//     bf16 (l the fp32 sum of the row's p), so the product below is normalised;
//   O^T[dim][row] = V^T (A: a dim's 8 keys through two transposing LDS reads
//     of the 288-byte V rows) x P^T (B: p straight from the softmax
//     registers; key order inside a 32-key step follows the accumulator
//     layout, and V follows it): with V's dims placed as below, a lane holds
//     row c16's dims 32 m + 8 grp .. +7 in tiles 2 m and 2 m + 1;
//   the wave's 16 rows of o / l (bf16) are exchanged through LDS and stored 4
//     whole rows per instruction, whole 128-byte lines (half-line stores of
//     the same bytes cost about 27 % more HBM writes and 6 % of the prefill).
// KV8: the caches hold E4M3 codes (one byte per element), turned into bf16
// (exactly) as they go to LDS; the scales and the rotation are in the
// softmax scale, the rotated query (ks_rotate_q_kernel) and the merge.
template <int G, int KT, bool KV8>
__global__ __launch_bounds__(256, 3) void ks_attn_kernel(Geo g, KsArgs a,
                                                        const uint16_t* __restrict__ q,
                                                        const uint16_t* __restrict__ kc,
                                                        const uint16_t* __restrict__ vc) {
  constexpr int D = 128, RB = 16 * KT;
  constexpr int KS = 272, VS = 288;
  constexpr int TQ = kRows / G;  // queries per tile
  typedef short v4s __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) unsigned char Kl[RB * KS];
  __shared__ __attribute__((aligned(16))) unsigned char Vl[RB * VS];
  __shared__ int32_t s_t[kKsItemMax], s_slot[kKsItemMax], s_p[kKsItemMax];
  __shared__ __attribute__((aligned(16))) uint4 Os[4][16 * 16];  // a wave's 16 output rows
  // Workgroups go round-robin over the 8 XCDs (blockIdx % 8).  When Hkv
  // divides 8, XCD x serves KV head x / (8 / Hkv) and items of its residue,
  // in item order: the items an XCD runs together read one query range.
  int item_idx, kvh;
  if (8 % g.Hkv == 0) {
    const int per = 8 / g.Hkv, x = blockIdx.x & 7;
    kvh = x / per;
    item_idx = (blockIdx.x >> 3) * per + (x - kvh * per);
  } else {
    item_idx = blockIdx.x / g.Hkv;
    kvh = blockIdx.x - item_idx * g.Hkv;
  }
  if (item_idx >= a.n_items) return;
  const int4 item = a.items[item_idx];
  const int cnt = item.z;
  if (cnt <= 0) return;
  const int tid = threadIdx.x;
  const int wid = tid >> 6, lane = tid & 63, c16 = lane & 15, grp = lane >> 4;
  const int l0 = item.x, j = item.y, b = item.w;
  const int past = g.past_len[b], cu0 = g.cu_q[b], cu1 = g.cu_q[b + 1];
  const int n_b = past + (cu1 - cu0);  // rows the sequence holds after this call
  const int key0 = j << g.log2r;
  const int h0 = kvh * G;

  if (tid < cnt) {
    const uint32_t e = a.list[l0 + tid];
    const int t = (int)(e >> kKsSlotBits);
    s_t[tid] = t;
    s_slot[tid] = (int)(e & ((1u << kKsSlotBits) - 1u));
    s_p[tid] = past + (t - cu0);
  }
  // The block's K and V rows to LDS (rows at or past the sequence's length,
  // or outside the cache, read as zero).
  if constexpr (KV8) {
    const uint8_t* k8 = reinterpret_cast<const uint8_t*>(kc);
    const uint8_t* v8 = reinterpret_cast<const uint8_t*>(vc);
    for (int cidx = tid; cidx < RB * 8; cidx += 256) {
      const int row = cidx >> 3, c8 = cidx & 7, s = key0 + row;  // dims 16 c8 .. +15
      const int64_t off = s < n_b ? kv_row(g, b, kvh, s) : -1;
      uint4 kw = *reinterpret_cast<const uint4*>(k8 + max(off, (int64_t)0) + 16 * c8);
      uint4 vw = *reinterpret_cast<const uint4*>(v8 + max(off, (int64_t)0) + 16 * c8);
      if (off < 0) kw = vw = make_uint4(0u, 0u, 0u, 0u);
      uint32_t kb[8], vb[8];
      const uint32_t kx[4] = {kw.x, kw.y, kw.z, kw.w}, vx[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kb[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kx[i], 1.0f, false));
        kb[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kx[i], 1.0f, true));
        vb[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vx[i], 1.0f, false));
        vb[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vx[i], 1.0f, true));
      }
      *reinterpret_cast<uint4*>(Kl + row * KS + 32 * c8) = make_uint4(kb[0], kb[1], kb[2], kb[3]);
      *reinterpret_cast<uint4*>(Kl + row * KS + 32 * c8 + 16) = make_uint4(kb[4], kb[5], kb[6], kb[7]);
      // V: 4-dim chunks 4 (c8 % 2) + i of the 32-dim group c8 / 2, placed as
      // below (chunk 2 c at position c, chunk 2 c + 1 at position 4 + c)
      unsigned char* vrow = Vl + row * VS + 64 * (c8 >> 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int cc = 4 * (c8 & 1) + i, pos = (cc & 1) ? 4 + (cc >> 1) : (cc >> 1);
        *reinterpret_cast<uint2*>(vrow + 8 * pos) = make_uint2(vb[2 * i], vb[2 * i + 1]);
      }
    }
  } else
  for (int cidx = tid; cidx < RB * 16; cidx += 256) {
    const int row = cidx >> 4, ch = cidx & 15, s = key0 + row;
    const int64_t off = s < n_b ? kv_row(g, b, kvh, s) : -1;
    // (unconditional loads at row 0 for rows that read as zero)
    uint4 kv = *reinterpret_cast<const uint4*>(kc + max(off, (int64_t)0) + 8 * ch);
    uint4 vv = *reinterpret_cast<const uint4*>(vc + max(off, (int64_t)0) + 8 * ch);
    if (off < 0) kv = vv = make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4*>(Kl + row * KS + 16 * ch) = kv;
    // V's 4-dim chunks are placed so that the two 16-dim MFMA tiles of each
    // 32 dims hand a lane 8 consecutive dims of its row: in dims 32 m .. 32 m
    // + 31, chunk 2 c sits at position c and chunk 2 c + 1 at position 4 + c.
    unsigned char* vrow = Vl + row * VS + 64 * (ch >> 2) + 8 * (ch & 3);
    *reinterpret_cast<uint2*>(vrow) = make_uint2(vv.x, vv.y);
    *reinterpret_cast<uint2*>(vrow + 32) = make_uint2(vv.z, vv.w);
  }
  __syncthreads();

  // This lane's row of tile c: its query, slot, position and query vector.
  const int R = 16 * wid + c16, u = R / G, hh = R - u * G;
  struct Row {
    int t, slot, p;
    uint4 qa[4];
  };
  auto load_row = [&](int c, Row& rw) {
    const int idx = c * TQ + u;
    rw.t = idx < cnt ? s_t[idx] : -1;
    rw.slot = idx < cnt ? s_slot[idx] : 0;
    rw.p = idx < cnt ? s_p[idx] : -1;
    // (unconditional loads: a row past the item's queries reads query 0's
    // heads, and its softmax is masked whole)
    const uint16_t* src =
        a.qrot != nullptr
            ? a.qrot + ((int64_t)(max(rw.t, a.t_lo) - a.t_lo) * g.Hq + h0 + hh) * D + 8 * grp
            : q + ((int64_t)max(rw.t, 0) * g.Hq + h0 + hh) * D + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) rw.qa[ks] = *reinterpret_cast<const uint4*>(src + 32 * ks);
  };
  const int n_tiles = (cnt + TQ - 1) / TQ;
  const f32x4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  auto run_tile = [&](const Row& rw) {
#ifdef QSA_COUNT_KEYS
    if (grp == 0 && rw.t >= 0 && hh == 0)
      atomicAdd(&g_ks_keys_visited, (unsigned long long)max(0, min(RB, rw.p - key0 + 1)));
#endif
    // S^T = K Q^T
    f32x4_t S[KT];
#pragma unroll
    for (int n = 0; n < KT; ++n) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 ka = *reinterpret_cast<const uint4*>(Kl + (16 * n + c16) * KS + 64 * ks + 16 * grp);
        S[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka),
                                                       __builtin_bit_cast(bf16x8_t, rw.qa[ks]),
                                                       ks == 0 ? zero4 : S[n], 0, 0, 0);
      }
    }
    // Softmax of row c16 over the keys it may see (the mask only where some
    // row of the wave cannot see the whole block: its tail block).
    // The maximum is taken over the raw scores (the scale is positive), and
    // the scale joins the exponent's argument: p = exp2(s c - m c).
    const int lim = rw.t >= 0 ? rw.p - key0 : -1;  // last visible key of the block
    const float sc = g.attn_scale_log2;
    float mx = -INFINITY;
    if (__all(lim >= RB - 1)) {
#pragma unroll
      for (int n = 0; n < KT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, S[n][r]);
    } else {
#pragma unroll
      for (int n = 0; n < KT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (16 * n + 4 * grp + r > lim) S[n][r] = -INFINITY;
          mx = fmaxf(mx, S[n][r]);
        }
    }
    mx = max_xor32(max_xor16(mx));
    // a row with no visible key: every p is 0 (exp2(-inf) = 0)
    const float mb = mx == -INFINITY ? 0.0f : mx * sc;
    // p / l rounded to bf16 for the matrix cores: the block's partial output
    // comes out normalised
    float pe[KT][4];
    float lsum = 0.0f;
#pragma unroll
    for (int n = 0; n < KT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pe[n][r] = __builtin_amdgcn_exp2f(fmaf(S[n][r], sc, -mb));
        lsum += pe[n][r];
      }
    const float l = sum_xor32(sum_xor16(lsum));
    const float inv = l > 0.0f ? __builtin_amdgcn_rcpf(l) : 0.0f;
    uint32_t pw[KT][2];
#pragma unroll
    for (int n = 0; n < KT; ++n)
#pragma unroll
      for (int h = 0; h < 2; ++h) pw[n][h] = pack_bf16(pe[n][2 * h] * inv, pe[n][2 * h + 1] * inv);
    // O^T = V^T P^T
    f32x4_t O[8];
#pragma unroll
    for (int ks = 0; ks < KT / 2; ++ks) {
      const unsigned char* v0 = Vl + (32 * ks + 4 * grp + (c16 >> 2)) * VS + 8 * (c16 & 3);
      const uint4 pb = make_uint4(pw[2 * ks][0], pw[2 * ks][1], pw[2 * ks + 1][0], pw[2 * ks + 1][1]);
#pragma unroll
      for (int nd = 0; nd < 8; ++nd) {
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(v0 + 32 * nd));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(v0 + 16 * VS + 32 * nd));
        const uint4 va = make_uint4(__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                                    __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y);
        O[nd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, va),
                                                        __builtin_bit_cast(bf16x8_t, pb),
                                                        ks == 0 ? zero4 : O[nd], 0, 0, 0);
      }
    }
    // Partial state of row c16: o (already divided by l) as bf16 (dims
    // 16 nd + 4 grp .. +3), and the base-2 log-sum-exp.
    // The wave's 16 rows go through LDS (16-byte chunks XOR-swizzled by
    // row) so that each store instruction writes 4 whole rows: 1 KB
    // contiguous when they are one query's heads.
    const int row = rw.t >= 0 ? ((rw.t - a.t_lo) * a.k1 + rw.slot) * g.Hq + h0 + hh : -1;
    uint4* os = Os[wid];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t w[4];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const f32x4_t& o = O[2 * m + x];
        w[2 * x] = pack_bf16(o[0], o[1]);
        w[2 * x + 1] = pack_bf16(o[2], o[3]);
      }
      os[c16 * 16 + ((4 * m + grp) ^ c16)] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    if (grp == 0 && row >= 0) a.pl[row] = l > 0.0f ? mb + __builtin_amdgcn_logf(l) : -INFINITY;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // (all four rows' indices and values read before the first store)
    int orow[4];
    uint4 ov[4];
    const int ch = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 4 * i + (lane >> 4);
      orow[i] = __shfl(row, rr, 64);
      ov[i] = os[rr * 16 + (ch ^ rr)];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (orow[i] >= 0)
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, ov[i]),
                                    reinterpret_cast<u32x4_t*>(a.po + (int64_t)orow[i] * D + 8 * ch));
    // (the next tile's writes to Os wait for these reads: in-order LDS
    // traffic of one wave)
    __builtin_amdgcn_wave_barrier();
  };
  // Two row buffers: the loads of tile c + 2 are requested once tile c is
  // done with its buffer, and arrive while tile c + 1 computes.
  Row ra, rb;
  load_row(0, ra);
  if (n_tiles > 1) load_row(1, rb);
  for (int c = 0; c < n_tiles; c += 2) {
    run_tile(ra);
    if (c + 2 < n_tiles) load_row(c + 2, ra);
    if (c + 1 >= n_tiles) break;
    run_tile(rb);
    if (c + 3 < n_tiles) load_row(c + 3, rb);
  }
}

// Log-sum-exp merge of a query's slots, then the gate.  One workgroup per
// (query, 16 heads); a thread takes 8 consecutive dims of one head (16-byte
// loads; a slot's 16 heads are 4 KB contiguous).  Slots: the query's
// selected blocks 0 .. n_blocks-1 (those whose entry names a candidate
// block: the plan made no entry for the others), then the tail (slot k)
// when it is not empty.  Every load of a round of kU slots is requested
// before the first is used; rounds merge under a running maximum.  Queries
// outside the capacities are left untouched, as the other attention kernels
// leave them.
__global__ __launch_bounds__(256) void ks_merge_kernel(Geo g, KsArgs a,
                                                      const int32_t* __restrict__ sel,
                                                      const int32_t* __restrict__ nblk,
                                                      const uint16_t* __restrict__ gate,
                                                      uint16_t* __restrict__ out) {
  constexpr int D = 128, kU = 12;
  const int tl = blockIdx.x, t = a.t_lo + tl;
  const int h = 16 * blockIdx.y + (threadIdx.x >> 4), d0 = 8 * (threadIdx.x & 15);
  if (h >= g.Hq) return;
  const QueryPos qp = query_pos(g, t);
  if (!qp.ok) return;
  const int64_t ob = ((int64_t)t * g.Hq + h) * D + d0;
  const uint4 gw = *reinterpret_cast<const uint4*>(gate + ob);
  const int n = qp.p + 1, nb = n >> g.log2r;
  const int nk = max(0, min(nblk[t], min(g.k, nb)));
  const bool tail = n > (nb << g.log2r);
  const int64_t row0 = (int64_t)tl * a.k1 * g.Hq + h;  // slot s: row0 + s * Hq
  const int n_slots = nk + (tail ? 1 : 0);
  const int32_t* srow = sel + (int64_t)t * g.k;
  float M = -INFINITY, den = 0.0f;
  float acc[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) acc[x] = 0.0f;
  for (int i0 = 0; i0 < n_slots; i0 += kU) {
    float lv[kU];
    uint4 ov[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = min(i0 + u, n_slots - 1);
      const int s = i < nk ? i : g.k;
      const int jb = i < nk ? srow[i] : 0;
      const int64_t row = row0 + (int64_t)s * g.Hq;
      const float lse = a.pl[row];
      ov[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                            reinterpret_cast<const u32x4_t*>(a.po + row * D + d0)));
      const bool valid = i0 + u < n_slots && (i >= nk || (jb >= 0 && jb < nb));
      lv[u] = valid ? lse : -INFINITY;
    }
    float cm = M;
#pragma unroll
    for (int u = 0; u < kU; ++u) cm = fmaxf(cm, lv[u]);
    // (the hardware exp2: exp2(-inf) = 0 for the invalid slots; a round with
    // none valid so far leaves everything at zero)
    const float sc = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - cm);
    den *= sc;
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[x] *= sc;
    const float cmv = cm == -INFINITY ? 0.0f : cm;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float w = __builtin_amdgcn_exp2f(lv[u] - cmv);
      const uint32_t wv[4] = {ov[u].x, ov[u].y, ov[u].z, ov[u].w};
      den += w;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        acc[2 * x] = fmaf(w, bf_lo(wv[x]), acc[2 * x]);
        acc[2 * x + 1] = fmaf(w, bf_hi(wv[x]), acc[2 * x + 1]);
      }
    }
    M = cm;
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
  for (int x = 0; x < 8; ++x) acc[x] *= inv;
  // 8-bit storage: the head's 16 threads un-rotate and scale the output
  // (every thread of a head is present: heads are whole 16-lane groups)
  if (g.kv8) kv8_output(g, acc, threadIdx.x & 15);
  const uint32_t gv[4] = {gw.x, gw.y, gw.z, gw.w};
  uint32_t o[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const float s0 = 1.0f / (1.0f + expf(-bf_lo(gv[x])));
    const float s1 = 1.0f / (1.0f + expf(-bf_hi(gv[x])));
    o[x] = (uint32_t)bf16_rne(acc[2 * x] * s0) | ((uint32_t)bf16_rne(acc[2 * x + 1] * s1) << 16);
  }
  *reinterpret_cast<uint4*>(out + ob) = make_uint4(o[0], o[1], o[2], o[3]);
}

template <int G, int KT, bool KV8>
void ks_launch_attn(const Geo& g, const KsArgs& a, int n_items, const void* q, const void* kc,
                    const void* vc, hipStream_t st) {
  // (8 % Hkv == 0: 8 workgroups per 8 / Hkv items, see the kernel)
  const int wgs = (8 % g.Hkv == 0) ? 8 * ((n_items + 8 / g.Hkv - 1) / (8 / g.Hkv)) : n_items * g.Hkv;
  ks_attn_kernel<G, KT, KV8><<<wgs, 256, 0, st>>>(
      g, a, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
      static_cast<const uint16_t*>(vc));
}

template <int G>
void ks_launch_g(const Geo& g, const KsArgs& a, int n_items, const void* q, const void* kc,
                 const void* vc, const int32_t* sel, const int32_t* nblk, const void* gate,
                 void* out, hipStream_t st) {
  if (g.kv8) {
    if (g.r == 32) ks_launch_attn<G, 2, true>(g, a, n_items, q, kc, vc, st);
    else if (g.r == 64) ks_launch_attn<G, 4, true>(g, a, n_items, q, kc, vc, st);
    else ks_launch_attn<G, 8, true>(g, a, n_items, q, kc, vc, st);
  } else {
    if (g.r == 32) ks_launch_attn<G, 2, false>(g, a, n_items, q, kc, vc, st);
    else if (g.r == 64) ks_launch_attn<G, 4, false>(g, a, n_items, q, kc, vc, st);
    else ks_launch_attn<G, 8, false>(g, a, n_items, q, kc, vc, st);
  }
  ks_merge_kernel<<<dim3(a.t_hi - a.t_lo, (g.Hq + 15) / 16), 256, 0, st>>>(
      g, a, sel, nblk, static_cast<const uint16_t*>(gate), static_cast<uint16_t*>(out));
}

}  // namespace

bool ks_supported(const Geo& g, int elem) {
  return elem == kBF16 && g.D == 128 && (g.r == 32 || g.r == 64 || g.r == 128) &&
         (g.G == 1 || g.G == 2 || g.G == 4 || g.G == 8 || g.G == 16) &&
         g.k + 1 <= (1 << kKsSlotBits);
}

int ks_item_tokens(const Geo&) { return kKsItemMax; }

int ks_groups(int64_t max_q, int64_t sub_tokens) {
  return (int)((std::min(max_q, sub_tokens) + kGroup - 1) / kGroup);
}

static int ks_ranges(int64_t max_q, int64_t sub_tokens) {
  return (ks_groups(max_q, sub_tokens) + kRangeGroups - 1) / kRangeGroups;
}

// Item slots of a sub-batch of n_tokens queries cut into nr query ranges per
// sequence: the end of the last sequence's region under item_base.
static int64_t ks_item_slots(const Geo& g, int nr, int64_t n_tokens) {
  const int64_t k1 = g.k + 1, nb1 = g.nbcap + 1;
  return n_tokens * k1 / ks_item_tokens(g) + (int64_t)g.B * (nr * nb1 + 1);
}

int64_t ks_item_bound(const Geo& g, int64_t max_q, int64_t sub_tokens) {
  return ks_item_slots(g, ks_ranges(max_q, sub_tokens), sub_tokens);
}

hipError_t launch_attend_ks(const Geo& g, const KsWork& w, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* sel, const int32_t* n_blocks,
                            const void* gate, void* out, hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  KsArgs a;
  a.k1 = g.k + 1;
  a.nb1 = g.nbcap + 1;
  a.item_tokens = ks_item_tokens(g);
  a.ng = ks_groups(w.max_q, w.sub_tokens);
  a.nr = ks_ranges(w.max_q, w.sub_tokens);
  if (w.sub_tokens > kKsSubTokens || a.nr > kMaxRanges) return hipErrorInvalidValue;
  a.list = w.list;
  a.items = w.items;
  a.hist = w.hist;
  a.boff = w.boff;
  a.po = w.po;
  a.pl = w.pl;
  a.qrot = g.rot ? w.qrot : nullptr;
  const size_t lds = (size_t)a.nb1 * sizeof(int32_t);
  for (int t_lo = 0; t_lo < g.T; t_lo += w.sub_tokens) {
    a.t_lo = t_lo;
    a.t_hi = std::min(g.T, t_lo + w.sub_tokens);
    // (a.nr, as the plan kernels' item_base uses it: a short last sub-batch
    // keeps the ranges of a full one)
    const int n_items = (int)ks_item_slots(g, a.nr, a.t_hi - a.t_lo);
    a.n_items = n_items;
    if (a.qrot != nullptr)
      ks_rotate_q_kernel<<<(int)(((int64_t)(a.t_hi - a.t_lo) * g.Hq + 15) / 16), 256, 0, st>>>(
          g, a, static_cast<const uint16_t*>(q));
    ks_count_kernel<<<dim3(a.ng, g.B), 256, lds, st>>>(g, a, sel, n_blocks);
    if (a.nb1 <= kScanThreads) {
      ks_scan_scatter_kernel<<<dim3(a.ng, g.B), kScanThreads, lds, st>>>(g, a, sel, n_blocks);
    } else {
      if (a.nb1 <= 2 * kScanThreads) ks_scan_kernel<2><<<g.B, kScanThreads, 0, st>>>(g, a);
      else if (a.nb1 <= 4 * kScanThreads) ks_scan_kernel<4><<<g.B, kScanThreads, 0, st>>>(g, a);
      else ks_scan_kernel<8><<<g.B, kScanThreads, 0, st>>>(g, a);
      ks_scatter_kernel<<<dim3(a.ng, g.B), 256, lds, st>>>(g, a, sel, n_blocks);
    }
    switch (g.G) {
      case 1: ks_launch_g<1>(g, a, n_items, q, k_cache, v_cache, sel, n_blocks, gate, out, st); break;
      case 2: ks_launch_g<2>(g, a, n_items, q, k_cache, v_cache, sel, n_blocks, gate, out, st); break;
      case 4: ks_launch_g<4>(g, a, n_items, q, k_cache, v_cache, sel, n_blocks, gate, out, st); break;
      case 8: ks_launch_g<8>(g, a, n_items, q, k_cache, v_cache, sel, n_blocks, gate, out, st); break;
      default: ks_launch_g<16>(g, a, n_items, q, k_cache, v_cache, sel, n_blocks, gate, out, st); break;
    }
  }
  return hipGetLastError();
}

#ifdef QSA_COUNT_KEYS
hipError_t ks_keys_visited(unsigned long long* value, bool reset) {
  hipError_t e = hipMemcpyFromSymbol(value, HIP_SYMBOL(g_ks_keys_visited), sizeof(*value));
  if (e != hipSuccess || !reset) return e;
  const unsigned long long zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_ks_keys_visited), &zero, sizeof(zero));
}
#endif

}  // namespace qsa
