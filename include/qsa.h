/*
 * qsa.h -- C ABI of the Qwen Sparse Attention (QSA) hot path on AMD Instinct
 * MI355X (gfx950).  Library: libqsa.so (HIP kernels, no host-side compute).
 *
 * What is computed (per query token t of sequence b at position p, n = p+1):
 *   1. Indexer keys are mean-pooled over complete blocks of r tokens
 *      ("mean-pooled key blocks": MTPLX "Native Backend Components for the
 *      Qwen4-Generation Preview Family", section "Qwen Sparse Attention").
 *   2. Each candidate block j < floor(n/r) is scored
 *        s_j = sum_h w[t,h] * relu(idx_scale * <q_idx[t,h], pooled_j>)
 *      (DeepSeek-style indexer logits with head scale 1 and softmax scale
 *      d_I^-0.5: llama.cpp PR #27739 page, LocalAI QSA-block commit, opening
 *      paragraph).
 *   3. The top k = budget / r blocks are kept (ties: lowest block index), plus
 *      the incomplete tail [r*floor(n/r), n), which is always kept (dev.to
 *      Qwen4-Exp article, section "Qwen Sparse Attention").  When
 *      floor(n/r) <= k every candidate is kept ("Porting Qwen4 to llama.cpp",
 *      section "QSA Should First Be Implemented as Selection Semantics").
 *   4. Every kept token is <= p (the causal intersection), and gated GQA
 *      softmax attention runs over exactly those tokens: query head h reads KV
 *      head h / (Hq/Hkv); out = softmax(attn_scale * q K^T) V * sigmoid(gate),
 *      elementwise ("selected block IDs -> direct indexed K/V loads -> online
 *      softmax -> output accumulation": same porting article, section "CUDA
 *      Optimization Should Follow State Correctness").
 *
 * Conventions shared by every entry point:
 *  - All pointers except the two structs are DEVICE pointers owned by the
 *    caller; the library never allocates, frees or keeps device memory, and
 *    holds no per-sequence state.  Save, restore and clone of the indexer
 *    state are the caller's copies of k_idx_cache and pooled.
 *  - stream is a hipStream_t (NULL = default stream).  Calls only enqueue
 *    work: no host synchronisation and no device-to-host reads.
 *  - Every argument is validated on the host BEFORE anything is enqueued; on
 *    error nothing is launched, a status < 0 is returned and qsa_last_error()
 *    gives the reason.  Device-side metadata (cu_q, past_len, page_table,
 *    sel, n_blocks) cannot be checked on the host; the kernels skip rows whose
 *    metadata falls outside the stated capacities instead of faulting.
 *  - n_tokens == 0 is a no-op returning QSA_OK.
 *  - Layouts (row-major, contiguous, element type = params.dtype unless said):
 *      q, gate, out         [T][Hq][D]
 *      k_new, v_new         [T][Hkv][D]
 *      q_idx                [T][H_I][d_I]
 *      k_idx_new            [T][d_I]
 *      w                    [T][H_I]                      fp32
 *      k_cache, v_cache     contiguous: [B][Hkv][kv_capacity][D]
 *                           paged:      [n_pages][Hkv][page_size][D]
 *                           (elements of params.kv_dtype)
 *      k_idx_cache          contiguous: [B][kv_capacity][d_I]
 *                           paged:      [n_pages][page_size][d_I]
 *      pooled               [B][d_I][pooled_ld]   fp32, column-major per
 *                           sequence (block j of dimension x at x*pooled_ld+j),
 *                           pooled_ld = qsa_pooled_ld(params, batch)
 *      sel                  [T][k] int32, ascending block ids, -1 padded
 *      n_blocks             [T] int32 = min(k, floor(n/r))
 *      scores               [T][max_kv_len / r] fp32, -inf past floor(n/r)
 *  - Token t belongs to sequence b with cu_q[b] <= t < cu_q[b+1]; its
 *    position is past_len[b] + (t - cu_q[b]).
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QSA_OK = 0,
  QSA_ERR_INVALID = -1,     /* bad argument or inconsistent sizes */
  QSA_ERR_UNSUPPORTED = -2, /* valid, but a shape this build has no kernel for */
  QSA_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than qsa_workspace_size */
  QSA_ERR_HIP = -4          /* a HIP launch failed; qsa_last_error has its text */
} qsa_status;

typedef enum { QSA_F32 = 0, QSA_BF16 = 1 } qsa_dtype;

/* Storage of the K/V caches ("Porting Qwen4 to llama.cpp", section "Quantized
 * KV Is a Representation Contract": quantized K/V may live in a
 * Hadamard-rotated basis, and a QSA attention path must honour that storage).
 *  QSA_KV_SAME: elements of params.dtype.
 *  QSA_KV_FP8:  one byte per element, OCP E4M3 (1 sign, 4 exponent bits with
 *               bias 7, 3 mantissa bits, no infinities, largest finite 448);
 *               a stored code c of K stands for e4m3(c) * k_scale, of V for
 *               e4m3(c) * v_scale.  With kv_rotate = 1 every stored row is
 *               H x, H the Sylvester Hadamard matrix of order D (entries
 *               +-1); the attention rotates the query and un-rotates its
 *               output (H o' / D), so results are those of the plain basis.
 *               The library encodes rows it appends: x (rotated if asked)
 *               times the fp32 value 1.0f / scale, rounded to the nearest code
 *               (ties to even), saturating at +-448. */
typedef enum { QSA_KV_SAME = 0, QSA_KV_FP8 = 2 } qsa_kv_dtype;

/* Layer geometry (host values). */
typedef struct {
  int32_t n_q_heads;   /* Hq, a multiple of n_kv_heads */
  int32_t n_kv_heads;  /* Hkv; Hq/Hkv in {1,2,4,8,16} */
  int32_t head_dim;    /* D in {64, 128} */
  int32_t n_idx_heads; /* H_I in [1, 16] */
  int32_t idx_dim;     /* d_I in {32, 64, 128} */
  int32_t block_size;  /* r, a power of two in [4, 256]; 0 = dense layer (ratio 0
                          marks a non-QSA layer: llama.cpp PR page, MTP commit) */
  int32_t ratio;       /* the pages' compression ratio; must equal block_size */
  int32_t budget;      /* tokens; k = budget / r in [1, 2048] (floor) */
  float attn_scale;    /* <= 0 selects D^-0.5 */
  float idx_scale;     /* <= 0 selects d_I^-0.5 */
  int32_t dtype;       /* qsa_dtype of q, k, v, gate, out, q_idx, k_idx */
  int32_t kv_dtype;    /* qsa_kv_dtype of k_cache / v_cache; QSA_KV_FP8 needs dtype
                          QSA_BF16 and D = 128 */
  int32_t kv_rotate;   /* QSA_KV_FP8 only: 1 = rows stored in the rotated basis
                          (needs Hq/Hkv >= 4) */
  float k_scale;       /* QSA_KV_FP8: scale of the K codes (> 0) */
  float v_scale;       /* QSA_KV_FP8: scale of the V codes (> 0) */
  int32_t idx_rope_dim;   /* rotary indexer keys: 0 = none; else an even number <= d_I.
                             Each pooled key's first idx_rope_dim values are rotated at
                             the block's first position j*r (rotate-half RoPE, frequencies
                             idx_rope_theta^(-2i/idx_rope_dim), angle and its cosine/sine
                             in fp64 rounded to fp32, rotation in fp32).  The caller's
                             q_idx must be rotated the same way at its own position
                             (qsa_block_forward does it).  LocalAI QSA-block commit: RoPE on
                             the indexer query and pooled keys, one set of angles. */
  float idx_rope_theta;   /* base of those frequencies (> 0 when idx_rope_dim > 0) */
} qsa_params;

/* One call's batch (host sizes for launch geometry + device metadata). */
typedef struct {
  int32_t n_seqs;      /* B >= 1 */
  int32_t n_tokens;    /* T = new tokens in this call, all sequences; >= 0 */
  int32_t max_q_len;   /* >= max_b (cu_q[b+1]-cu_q[b]) */
  int32_t max_kv_len;  /* >= max_b past_len[b] + new tokens of b */
  int32_t kv_capacity; /* rows per sequence; paged: max_pages * page_size */
  int32_t page_size;   /* 0 = contiguous caches; else a power of two */
  int32_t max_pages;   /* columns of page_table (paged) */
  int32_t n_pages;     /* physical pages in the cache pool (paged) */
  const int32_t* cu_q;       /* [B+1] device, cu_q[0] = 0, cu_q[B] = T */
  const int32_t* past_len;   /* [B] device, rows cached before this call */
  const int32_t* page_table; /* [B][max_pages] device physical page ids, or NULL */
} qsa_batch;

/* Text of the last failure on the calling thread ("" if none). */
const char* qsa_last_error(void);

/* Leading dimension of the pooled cache: ceil(kv_capacity / r) rounded up to a
 * multiple of 64.  Returns 0 for a dense layer or invalid arguments. */
int64_t qsa_pooled_ld(const qsa_params* params, const qsa_batch* batch);

/* Bytes of scratch workspace any entry point may need for this call (same
 * value for every entry point; 0 when n_tokens == 0).  The workspace holds
 * block scores, split-attention partials and, when the caller does not ask
 * for them, the selections.  Its contents need no initialisation; calls that
 * share one workspace must not overlap in time (same stream, or synchronised). */
size_t qsa_workspace_size(const qsa_params* params, const qsa_batch* batch);

/* Indexer-key append and incremental block pooling.
 * Writes k_idx_new[t] to k_idx_cache row past_len[b] + (t - cu_q[b]) (row
 * past_len, not row 0: LocalAI QSA-block commit, section "The battery"), then
 * pools every block completed by this call:
 *   pooled_j[x] = (sum over s = jr .. jr+r-1, ascending, of k_idx[s][x]) / r
 * in fp32.  Only new blocks are touched, O(new tokens) -- not the whole-cache
 * recompute of the upstream reference ("The trap the layer loop walks into").
 * Dense layer (block_size 0): QSA_ERR_INVALID. */
qsa_status qsa_pool_keys(const qsa_params* params, const qsa_batch* batch,
                         const void* k_idx_new, void* k_idx_cache, float* pooled,
                         void* stream);

/* K/V append only: writes k_new[t], v_new[t] to rows past_len[b] + (t -
 * cu_q[b]) of k_cache / v_cache under the layer's storage (QSA_KV_FP8: rotated
 * if asked, scaled and encoded as above).  For filling a cache with context
 * rows; qsa_forward appends its own new rows. */
qsa_status qsa_store_kv(const qsa_params* params, const qsa_batch* batch, const void* k_new,
                        const void* v_new, void* k_cache, void* v_cache, void* stream);

/* Block scoring and top-k selection (steps 2-3 above).
 * Reads q_idx [T][H_I][d_I], w [T][H_I] and the pooled cache; writes sel and
 * n_blocks; scores_opt (may be NULL) receives the pre-top-k scores, the value
 * gate of the LocalAI QSA-block commit.  ws: qsa_workspace_size bytes. */
qsa_status qsa_score_select(const qsa_params* params, const qsa_batch* batch,
                            const void* q_idx, const float* w, const float* pooled,
                            int32_t* sel, int32_t* n_blocks, float* scores_opt, void* ws,
                            size_t ws_bytes, void* stream);

/* Gated GQA attention over the selected blocks plus the tail (step 4).
 * The caches must already hold every token up to each query's position.
 * sel / n_blocks as written by qsa_score_select (ignored for a dense layer,
 * which attends all of [0, n)).  out [T][Hq][D]. */
qsa_status qsa_attend(const qsa_params* params, const qsa_batch* batch, const void* q,
                      const void* k_cache, const void* v_cache, const int32_t* sel,
                      const int32_t* n_blocks, const void* gate, void* out, void* ws,
                      size_t ws_bytes, void* stream);

/* The whole QSA layer step for one batch of new tokens: append k_new, v_new,
 * k_idx_new to the caches at each sequence's past_len, pool the completed
 * blocks, score, select, and attend.  sel_opt / n_blocks_opt (may be NULL)
 * receive the selections.  A dense layer skips the indexer. */
qsa_status qsa_forward(const qsa_params* params, const qsa_batch* batch, const void* q,
                       const void* k_new, const void* v_new, const void* q_idx,
                       const void* k_idx_new, const float* w, const void* gate,
                       void* k_cache, void* v_cache, void* k_idx_cache, float* pooled,
                       void* out, int32_t* sel_opt, int32_t* n_blocks_opt, void* ws,
                       size_t ws_bytes, void* stream);

/* qsa_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same launches on the same kernels, with the workspace taken from a scratch
 * array inside the library instead of a ws argument.  Arguments, results
 * and errors as qsa_forward.
 *   - The scratch holds QSA_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, allocated
 *     with the library's code on each device it runs on and held until the
 *     process ends; a call whose qsa_workspace_size exceeds it returns
 *     QSA_ERR_WORKSPACE and launches nothing.
 *   - No device memory is allocated or freed, by the library or by any
 *     routine it calls; nothing in the scratch has to start at zero (every
 *     value a call reads there, that call wrote first).
 *   - The scratch is looked up on the calling thread's current device, which
 *     must be the device of `stream`.
 *   - All calls on one GPU share its scratch: calls that overlap in time on
 *     one GPU (different streams, or different host threads without
 *     ordering) race and give undefined results; calls ordered on one
 *     stream are fine. */
#define QSA_NOALLOC_SCRATCH_BYTES (16u << 20)
qsa_status qsa_forward_noalloc(const qsa_params* params, const qsa_batch* batch, const void* q,
                               const void* k_new, const void* v_new, const void* q_idx,
                               const void* k_idx_new, const float* w, const void* gate,
                               void* k_cache, void* v_cache, void* k_idx_cache, float* pooled,
                               void* out, int32_t* sel_opt, int32_t* n_blocks_opt,
                               void* stream);

/* ------------------------------------------------------------------------
 * The QSA attention block around the path (llama.cpp PR #27739 page,
 * LocalAI QSA-block commit, opening paragraph: q/k/v/o projections, the
 * (1 + w) q/k norms, RoPE, the indexer, the gather consumer, the sigmoid
 * output gate and o_proj; fresh-review section: one set of rotary angles for
 * the query side and the pooled indexer keys).
 *
 * Readings where the pages are silent:
 *   - weights are Linear [out][in] bf16; w_in stacks the rows of the q (Hq*D),
 *     gate (Hq*D), k (Hkv*D), v (Hkv*D), indexer-query (H_I*d_I) and
 *     indexer-key (d_I) projections, in that order (a dense layer has no
 *     indexer rows); w_o is [d_model][Hq*D];
 *   - q/k norm: RMSNorm over each head's D values, x / sqrt(mean(x^2) + eps)
 *     * (1 + w) with one [D] bf16 weight shared by the heads;
 *   - RoPE (rotate-half) on the first rotary_dim values of each q and k head
 *     at the token's position; the indexer query with idx_rope_dim /
 *     idx_rope_theta of qsa_params, the pooled keys as documented there;
 *   - indexer head weights all ones, no indexer norm; the gate is its own
 *     projection, sigmoid-applied elementwise. */
typedef struct {
  int32_t d_model;     /* hidden size, a multiple of 32 */
  int32_t rotary_dim;  /* rotated values per q/k head, even, <= head_dim */
  float rope_theta;    /* RoPE base (> 0 when rotary_dim > 0) */
  float norm_eps;      /* RMSNorm epsilon (>= 0) */
} qsa_block_params;

/* Workspace bytes of qsa_block_forward for this call (0 on invalid
 * arguments or n_tokens == 0). */
size_t qsa_block_workspace_size(const qsa_params* params, const qsa_block_params* block,
                                const qsa_batch* batch);

/* One QSA block step for the batch's new tokens: x [T][d_model] bf16 hidden
 * states -> y [T][d_model] bf16.  Projections on bf16 matrix cores with fp32
 * accumulation; q, gate, k, v, indexer q and k rounded to bf16 after the
 * norm and RoPE; then the QSA step of qsa_forward (append K/V and indexer
 * keys at past_len, pool, score, select, attend, gate) on those tensors;
 * then o_proj of the bf16 attention output.  q_norm / k_norm: [D] bf16.
 * Caches, pooled cache, selections and errors as qsa_forward; ws:
 * qsa_block_workspace_size bytes, 16-byte aligned.  dtype must be QSA_BF16. */
qsa_status qsa_block_forward(const qsa_params* params, const qsa_block_params* block,
                             const qsa_batch* batch, const void* x, const void* w_in,
                             const void* q_norm, const void* k_norm, const void* w_o,
                             void* k_cache, void* v_cache, void* k_idx_cache, float* pooled,
                             void* y, int32_t* sel_opt, int32_t* n_blocks_opt, void* ws,
                             size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
