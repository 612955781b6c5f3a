// Internal interface between the C-ABI host layer (qsa_api.hip) and the
// gfx950 kernels (qsa_kernels.hip, qsa_prefill_ks.hip, qsa_block.hip) and the
// library GEMM path (qsa_blas.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// Per-call geometry, passed to every kernel by value.
struct Geo {
  int32_t Hq, Hkv, G, D;       // query heads, KV heads, heads per KV head, head dim
  int32_t HI, dI;              // indexer heads and dim
  int32_t r, log2r, k;         // block size (0 = dense), log2, blocks kept
  int32_t B, T;                // sequences, new tokens
  int32_t one_q;               // 1: every sequence has exactly one new token (t = b)
  int32_t cap;                 // rows per sequence
  int32_t page_size, log2ps;   // 0 = contiguous
  int32_t max_pages, n_pages;
  int32_t pooled_ld;           // leading dim of the pooled cache
  int32_t nbcap;               // row stride of the score buffer (max_kv_len / r)
  float attn_scale_log2;       // attn_scale * log2(e): softmax runs in base 2
  float idx_scale;             // indexer softmax scale (fp32, applied as c * d)
  float inv_r;                 // 1 / r, exact because r is a power of two
  int32_t kv8;                 // 1: K/V caches hold OCP E4M3 codes (one byte per element)
  int32_t rot;                 // 1: ... in the Sylvester-Hadamard-rotated basis
  int32_t kv_esz;              // bytes per K/V cache element
  float inv_k_scale, inv_v_scale;  // 8-bit: 1 / scale, the factor applied before encoding
  float out_scale;             // 8-bit: V scale (and 1/D when rotated) on the attention output
  int32_t idx_rope_dim;        // > 0: each pooled key's first idx_rope_dim values are rotated
                               // at its block's first position (frequencies: RopeTab)
  const int32_t* cu_q;
  const int32_t* past_len;
  const int32_t* page_table;
};

// Rotary frequencies theta^(-2i/R), fp64, computed on the host.  Kept out of
// Geo and passed only to the kernels that rotate: a 512-byte table inside
// Geo costs every kernel scalar registers.
struct RopeTab {
  double f[64];
};

// Split-KV plan of the attention kernels.
struct AttnPlan {
  int32_t ks;            // 1: key-stationary prefill path (launch_attend_ks)
  int32_t mfma;          // 1: prefill MFMA kernel (one wave per unit, no splits)
  int32_t n_splits;      // splits per (token, KV head), <= kPlanMaxSplits
  int32_t tiles;         // 64-token tiles of the longest selection list
};
constexpr int kPlanMaxSplits = 128;
constexpr int kPlanMaxK = 2048;  // budget / block_size
constexpr int kSelectInKernelMaxBlocks = 2048;  // candidate blocks the in-kernel selection holds

// Waves per workgroup of the attention kernel chosen for this dtype / head dim.
inline int attend_waves(int elem, int D) { return (elem == 1 && D == 128) ? 4 : 1; }

enum ElemType { kF32 = 0, kBF16 = 1 };

// Launchers; each returns hipGetLastError() after its launches.
hipError_t launch_append_pool(const Geo& g, int elem, const void* k_new, const void* v_new,
                              const void* kI_new, void* k_cache, void* v_cache, void* kI_cache,
                              float* pooled, const RopeTab& idx_rope, hipStream_t st);
hipError_t launch_score(const Geo& g, int elem, const void* qI, const float* w, float* pooled,
                        float* scores, hipStream_t st);
// Rows a decode-form score launch appends (at most one new token per sequence).
struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const void* kI_new;
  void* k_cache;
  void* v_cache;
  void* kI_cache;
};
hipError_t launch_score_append(const Geo& g, int elem, const void* qI, const float* w,
                               float* pooled, float* scores, const AppendArgs& ap,
                               const RopeTab& idx_rope, hipStream_t st);
hipError_t launch_select(const Geo& g, const float* scores, int32_t* sel, int32_t* n_blocks,
                         hipStream_t st);
// In-kernel selection (decode attention): scores in, selections out (either
// output may be null).  scores == null: the selection is read from sel.
struct InKernelSelect {
  const float* scores;
  int32_t* sel_out;
  int32_t* n_blocks_out;
};
hipError_t launch_attend(const Geo& g, int elem, const AttnPlan& plan, const void* q,
                         const void* k_cache, const void* v_cache, const int32_t* sel,
                         const int32_t* n_blocks, const void* gate, void* out, float* part,
                         hipStream_t st, const InKernelSelect& fs = InKernelSelect{});

// The block front end (projections, norms, RoPE) and o_proj.
struct BlockPrepArgs {
  const float* part;           // [S][T][n_in] fp32 partials of the stacked input projection
  int32_t S, n_in;
  float eps;                   // RMSNorm epsilon
  int32_t rotary_dim;          // rotated values of each q / k head (rotate-half)
  double freq[64];             // their frequencies theta^(-2i/rotary_dim), fp64
  double idx_freq[64];         // the indexer query's (qsa_params idx_rope_dim / theta)
  const uint16_t* q_norm;      // [D] bf16, applied as (1 + w)
  const uint16_t* k_norm;
  uint16_t* q;                 // [T][Hq][D] bf16 outputs
  uint16_t* gate;              // [T][Hq][D]
  uint16_t* k;                 // [T][Hkv][D]
  uint16_t* v;                 // [T][Hkv][D]
  uint16_t* q_idx;             // [T][H_I][d_I]
  uint16_t* k_idx;             // [T][d_I]
  float* w;                    // [T][H_I], all ones
};
// Split count and k range per split of a projection GEMM of M x N x K.
int gemm_splits(int M, int N, int K);
int gemm_k_split(int K, int S);
// part: [S][M][N] fp32 partials; with S == 1 and out_bf16 given, the result
// goes straight to out_bf16 [M][N] instead.
hipError_t launch_proj_gemm(const void* A, const void* B, float* part, void* out_bf16, int M,
                            int N, int K, int S, hipStream_t st);
hipError_t launch_proj_reduce(const float* part, int S, int64_t MN, void* out, hipStream_t st);
// D[M][N] = A[M][K] · B[N][K]ᵀ on hipBLASLt (qsa_blas.hip); hipErrorNotSupported
// when it cannot run the product (the caller then runs its own kernel).
hipError_t lt_gemm(const void* A, const void* B, void* D, bool d_f32, int M, int N, int K,
                   hipStream_t st);
#ifdef QSA_COUNT_KEYS
// Debug builds: false makes lt_gemm decline every product (the tiled kernel runs).
void lt_set_enabled(bool on);
#endif
hipError_t launch_block_prep(const Geo& g, const BlockPrepArgs& a, hipStream_t st);

#ifdef QSA_COUNT_KEYS
// Debug builds: the device counter of K/V rows the attention kernels loaded
// (synchronous copies; reset sets it to zero after reading).
hipError_t keys_visited(unsigned long long* value, bool reset);
#endif

// True when a kernel instantiation exists for G heads per KV head and dim D.
bool attend_supported(int G, int D);

// Key-stationary prefill attention (qsa_prefill_ks.hip): per sub-batch of
// queries, a plan launch sorts the selection entries by block, an attention
// launch runs each block's queries through the block's K/V once, and a merge
// launch combines each query's per-block partial states.
constexpr int kKsSlotBits = 12;       // an entry packs (query << 12 | slot): k + 1 <= 4096
constexpr int kKsMaxBlocks = 8192;    // candidate blocks + 1 that one plan workgroup holds
constexpr int kKsMinQueries = 512;    // new tokens of one sequence that make the path pay
constexpr int kKsSubTokens = 4096;    // queries per sub-batch (bounds the partial buffers)
constexpr int kKsItemMax = 128;       // queries per work item of the attention
constexpr int kKsMaxSlots = 128;      // k + 1 the path takes
struct KsArgs {
  int32_t t_lo, t_hi;    // the sub-batch's queries [t_lo, t_hi)
  int32_t k1, nb1;       // slots per query (k + 1: the tail is slot k); blocks + 1
  int32_t item_tokens;   // queries per work item
  int32_t ng;            // counting groups per sequence
  int32_t nr;            // query ranges per sequence (of the work-item order)
  int32_t n_items;       // work-item slots of this sub-batch
  uint32_t* list;        // [sub * k1] entries, grouped by block
  int32_t* hist;         // [B][ng][nb1] entries per (group, block); after the scan, per
                         // (group, block) the entries of the block from earlier groups
  int32_t* boff;         // [B][nb1] first list position of each block
  int4* items;           // [ks_item_bound] work items {list start, block, count, sequence}
  uint16_t* po;          // [sub][k1][Hq][D] bf16 partial outputs, normalised
  float* pl;             // [sub][k1][Hq] base-2 log-sum-exp of each partial
  uint16_t* qrot;        // [sub][Hq][D] rotated queries (8-bit rotated caches), else null
};
struct KsWork {
  uint32_t* list;
  int4* items;
  int32_t* hist;
  int32_t* boff;
  uint16_t* po;
  float* pl;
  uint16_t* qrot;        // [sub][Hq][D] (8-bit rotated caches)
  int32_t sub_tokens;
  int32_t max_q;         // the batch's longest new-token count
};
bool ks_supported(const Geo& g, int elem);
int ks_item_tokens(const Geo& g);
int64_t ks_item_bound(const Geo& g, int64_t max_q, int64_t sub_tokens);
int ks_groups(int64_t max_q, int64_t sub_tokens);
hipError_t launch_attend_ks(const Geo& g, const KsWork& w, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* sel, const int32_t* n_blocks,
                            const void* gate, void* out, hipStream_t st);
#ifdef QSA_COUNT_KEYS
hipError_t ks_keys_visited(unsigned long long* value, bool reset);
#endif

}  // namespace qsa
