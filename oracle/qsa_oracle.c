/*
 * Qwen Sparse Attention (QSA) -- plain CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * statement of what the QSA hot path computes.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg load it; the product path
 * never does.  It shares no code, header, table or constant with the HIP
 * library.
 *
 * What it follows (pages of the Qwen4-Exp / Qwen3.8-Flash-Next material):
 *  - "Native Backend Components for the Qwen4-Generation Preview Family in
 *    MTPLX", section "Qwen Sparse Attention (QSA)": standard gated GQA whose
 *    causal mask is intersected with a per-query selection from a
 *    DeepSeek-V3.2-style indexer that relu-scores mean-pooled key blocks and
 *    keeps the top budget/ratio blocks plus the incomplete tail block.
 *  - "Qwen4-Exp: How Per-Layer N-gram Embeddings and Sparse Attention Are
 *    Reshaping Hybrid LLM Architecture", section "Qwen Sparse Attention":
 *    block-level selection; the trailing incomplete block is always kept.
 *  - llama.cpp PR #27739 page, LocalAI QSA-block commit, opening paragraph:
 *    the indexer is DeepSeek-style logits with all-ones head weights, head
 *    scale 1, softmax scale index_head_dim^-0.5 and candidate window
 *    kv_len / compress_ratio; the sigmoid output gate follows attention.
 *  - "Porting Qwen4 to llama.cpp: Qwen3.8-Flash-Next Internals", section
 *    "QSA Should First Be Implemented as Selection Semantics": selector ->
 *    blocks -> cache cells -> attention over the selected memory; width bound
 *    min(n_kv, budget + ratio - 1); dense equality at or below the budget.
 *
 * Precision: pooling and block scores are fp32 in the fixed order written
 * below (the order is part of the definition, because the scores decide an
 * integer selection and both sides must take that decision in the same
 * precision); ties are broken by the lowest block index.  Attention is
 * accumulated in fp64 and rounded to fp32 once at the end.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC
 * (no contraction, so every fp32 rounding is the one written here).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int32_t n_q_heads;   /* Hq */
  int32_t n_kv_heads;  /* Hkv; query head h reads KV head h / (Hq/Hkv) */
  int32_t head_dim;    /* D */
  int32_t n_idx_heads; /* H_I */
  int32_t idx_dim;     /* d_I */
  int32_t block_size;  /* r; 0 = dense layer (no selection) */
  int32_t budget;      /* tokens; k = budget / r complete blocks */
  float attn_scale;    /* <= 0: 1/sqrt(D) */
  float idx_scale;     /* <= 0: 1/sqrt(d_I) */
  int32_t idx_rope_dim;  /* > 0: rotary dims of each pooled key (see qsa_oracle_rope) */
  float idx_rope_theta;  /* base of those rotary frequencies */
} qsa_oracle_dims;

int qsa_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads of the calling thread's later parallel regions (the baseline's
 * single-core timing); 0 leaves the setting as it is. */
void qsa_oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Mean-pooled indexer key of every complete block ("mean-pooled key blocks",
 * MTPLX page, QSA section).  Column x of block j is the fp32 sum of
 * kI[j*r + s][x] for s = 0..r-1 in ascending order, divided by r.
 * Returns the number of complete blocks, floor(n_tok / r). */
int64_t qsa_oracle_pool(const float* kI, int64_t n_tok, int32_t d_idx, int32_t r,
                        float* pooled) {
  int64_t nb = n_tok / r;
  for (int64_t j = 0; j < nb; ++j) {
    for (int32_t x = 0; x < d_idx; ++x) {
      float acc = 0.0f;
      for (int32_t s = 0; s < r; ++s) acc = acc + kI[(j * r + s) * d_idx + x];
      pooled[j * d_idx + x] = acc / (float)r;
    }
  }
  return nb;
}

/* Rotary position embedding in the rotate-half form on the first R entries
 * of x (R even; the entries from R on are left alone), at position pos with
 * base theta.  For i < R/2 the pair (x[i], x[i + R/2]) turns by the angle
 * pos * f_i with f_i = theta^(-2i/R):
 *   x'[i] = x[i]*c - x[i+R/2]*s,   x'[i+R/2] = x[i+R/2]*c + x[i]*s.
 * f_i = pow(theta, -2i/R) and the angle are fp64, c and s are the fp64
 * cosine and sine rounded to fp32, and the rotation is fp32 (each product
 * rounded, then the sum).  (LocalAI QSA-block commit, opening paragraph:
 * the block applies RoPE after the q/k norms; fresh-review section: the
 * indexer query and the pooled indexer keys are rotated with the same
 * angles.) */
void qsa_oracle_rope(float* x, int32_t R, double theta, int64_t pos) {
  const int32_t h = R / 2;
  for (int32_t i = 0; i < h; ++i) {
    const double f = pow(theta, -2.0 * (double)i / (double)R);
    const double ang = (double)pos * f;
    const float c = (float)cos(ang), sn = (float)sin(ang);
    const float a = x[i], b = x[i + h];
    x[i] = a * c - b * sn;
    x[i + h] = b * c + a * sn;
  }
}

/* qsa_oracle_rope on `rows` rows of n entries, row i at position pos[i]. */
void qsa_oracle_rope_rows(float* x, int64_t rows, int32_t n, int32_t R, double theta,
                          const int64_t* pos) {
  for (int64_t i = 0; i < rows; ++i) qsa_oracle_rope(x + i * n, R, theta, pos[i]);
}

/* Relu-weighted multi-head block score (DeepSeek-style indexer logits with
 * head scale 1; LocalAI QSA-block commit, opening paragraph):
 *   s_j = sum_h w_h * relu(c * <qI_h, pooled_j>)
 * fp32; per head the dot product is a chain of fmaf over x ascending, then
 * a = c*d, relu (a non-positive a becomes +0), then s = fmaf(w_h, a, s),
 * heads ascending. */
void qsa_oracle_scores(const float* qI, const float* w, const float* pooled, int64_t nb,
                       int32_t n_idx_heads, int32_t d_idx, float c, float* s_out) {
  for (int64_t j = 0; j < nb; ++j) {
    const float* kb = pooled + j * d_idx;
    float s = 0.0f;
    for (int32_t h = 0; h < n_idx_heads; ++h) {
      const float* qh = qI + (int64_t)h * d_idx;
      float d = 0.0f;
      for (int32_t x = 0; x < d_idx; ++x) d = fmaf(qh[x], kb[x], d);
      float a = c * d;
      a = (a > 0.0f) ? a : 0.0f;
      s = fmaf(w[h], a, s);
    }
    s_out[j] = s;
  }
}

typedef struct {
  float s;
  int32_t j;
} scored_block;

/* Total order of the selection: higher score first, then lower index. */
static int by_score_then_index(const void* pa, const void* pb) {
  const scored_block* a = (const scored_block*)pa;
  const scored_block* b = (const scored_block*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->j < b->j) ? -1 : (a->j > b->j);
}

static int ascending_i32(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

/* Top-(budget/ratio) complete blocks among the nb candidates (MTPLX page, QSA
 * section; dev.to article, QSA section).  When nb <= k every candidate is
 * kept (the dense regime of the llama.cpp porting article, "QSA Should First
 * Be Implemented as Selection Semantics").  Otherwise candidates are sorted by
 * (score desc, index asc) and the first k kept.  Output ascending. */
int32_t qsa_oracle_topk(const float* s, int64_t nb, int32_t k, int32_t* sel) {
  if (nb <= k) {
    for (int64_t j = 0; j < nb; ++j) sel[j] = (int32_t)j;
    return (int32_t)nb;
  }
  scored_block* all = (scored_block*)malloc(sizeof(scored_block) * (size_t)nb);
  for (int64_t j = 0; j < nb; ++j) {
    all[j].s = s[j];
    all[j].j = (int32_t)j;
  }
  qsort(all, (size_t)nb, sizeof(scored_block), by_score_then_index);
  for (int32_t i = 0; i < k; ++i) sel[i] = all[i].j;
  free(all);
  qsort(sel, (size_t)k, sizeof(int32_t), ascending_i32);
  return k;
}

/* Token set of a query at position p (n = p + 1 visible tokens): the tokens
 * of every selected block plus the incomplete tail [r*nb, n), with
 * nb = floor(n / r).  Every token is <= p: this is the intersection with the
 * causal mask.  Dense layer (r == 0): all of [0, n).  Ascending. */
int64_t qsa_oracle_token_set(const int32_t* sel, int32_t n_sel, int32_t r, int64_t p,
                             int64_t* tokens) {
  int64_t n = p + 1, c = 0;
  if (r == 0) {
    for (int64_t t = 0; t < n; ++t) tokens[c++] = t;
    return c;
  }
  int64_t nb = n / r;
  for (int32_t i = 0; i < n_sel; ++i)
    for (int32_t s = 0; s < r; ++s) tokens[c++] = (int64_t)sel[i] * r + s;
  for (int64_t t = nb * r; t < n; ++t) tokens[c++] = t;
  return c;
}

/* Gated GQA softmax attention of one query over a token list (MTPLX page,
 * QSA section: "standard gated GQA"; LocalAI commit: gather consumer, then
 * the sigmoid output gate).  K, V: [n_tok][Hkv][D].  For head h, KV head
 * h / (Hq/Hkv); z_t = scale * <q_h, K_t>; softmax over the list; o = sum p V;
 * out = o * sigmoid(gate), elementwise (gate NULL: no gate).  fp64 accumulation. */
void qsa_oracle_attend(const float* q, const float* K, const float* V, const float* gate,
                       const int64_t* tokens, int64_t n_t, int32_t Hq, int32_t Hkv, int32_t D,
                       double scale, float* out) {
  int32_t g = Hq / Hkv;
  double* z = (double*)malloc(sizeof(double) * (size_t)(n_t > 0 ? n_t : 1));
  double* o = (double*)malloc(sizeof(double) * (size_t)D);
  for (int32_t h = 0; h < Hq; ++h) {
    int32_t kvh = h / g;
    const float* qh = q + (int64_t)h * D;
    double m = -INFINITY;
    for (int64_t i = 0; i < n_t; ++i) {
      const float* kr = K + (tokens[i] * Hkv + kvh) * D;
      double acc = 0.0;
      for (int32_t x = 0; x < D; ++x) acc += (double)qh[x] * (double)kr[x];
      z[i] = scale * acc;
      if (z[i] > m) m = z[i];
    }
    double l = 0.0;
    for (int32_t x = 0; x < D; ++x) o[x] = 0.0;
    for (int64_t i = 0; i < n_t; ++i) {
      double e = exp(z[i] - m);
      l += e;
      const float* vr = V + (tokens[i] * Hkv + kvh) * D;
      for (int32_t x = 0; x < D; ++x) o[x] += e * (double)vr[x];
    }
    for (int32_t x = 0; x < D; ++x) {
      double gt = gate ? 1.0 / (1.0 + exp(-(double)gate[(int64_t)h * D + x])) : 1.0;
      out[(int64_t)h * D + x] = (float)(o[x] / l * gt);
    }
  }
  free(z);
  free(o);
}

static float default_scale(float given, int32_t dim) {
  return given > 0.0f ? given : (float)(1.0 / sqrt((double)dim));
}

/* QSA for nq queries of ONE sequence.
 *   K, V      [n_tok][Hkv][D]   the sequence's keys/values (fp32 values)
 *   kI        [n_tok][d_I]      indexer keys
 *   pos       [nq]              query positions (each < n_tok)
 *   q, gate   [nq][Hq][D];  qI [nq][H_I][d_I];  w [nq][H_I]
 * Outputs:
 *   out       [nq][Hq][D]
 *   sel       [nq][k] ascending block ids, -1 padded (NULL allowed; k = budget/r)
 *   n_blocks  [nq] selected complete blocks (NULL allowed)
 *   n_tokens  [nq] size of the token set (NULL allowed)
 *   scores    [nq][nb_cap] block scores, -inf past the query's nb (NULL allowed)
 * Queries are independent; OpenMP spreads them over threads, so results do
 * not depend on the thread count.  Returns 0, or -1 on bad arguments. */
int qsa_oracle_sequence(const qsa_oracle_dims* dm, int64_t n_tok, const float* K,
                        const float* V, const float* kI, int64_t nq, const int64_t* pos,
                        const float* q, const float* qI, const float* w, const float* gate,
                        float* out, int32_t* sel, int32_t* n_blocks, int64_t* n_tokens,
                        float* scores, int64_t nb_cap) {
  const int32_t Hq = dm->n_q_heads, Hkv = dm->n_kv_heads, D = dm->head_dim;
  const int32_t HI = dm->n_idx_heads, dI = dm->idx_dim, r = dm->block_size;
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || r < 0) return -1;
  const int32_t k = r > 0 ? dm->budget / r : 0;
  if (r > 0 && (k < 1 || HI <= 0 || dI <= 0)) return -1;
  if (dm->idx_rope_dim < 0 || dm->idx_rope_dim % 2 || dm->idx_rope_dim > dI) return -1;
  for (int64_t i = 0; i < nq; ++i)
    if (pos[i] < 0 || pos[i] >= n_tok) return -1;
  const double a_scale = dm->attn_scale > 0.0f ? (double)dm->attn_scale
                                               : 1.0 / sqrt((double)D);
  const float c_idx = default_scale(dm->idx_scale, dI);

  float* pooled = NULL;
  if (r > 0) {
    pooled = (float*)malloc(sizeof(float) * (size_t)((n_tok / r) * dI + 1));
    const int64_t nbt = qsa_oracle_pool(kI, n_tok, dI, r, pooled);
    /* With rotary indexer keys, the pooled key of block j is rotated at the
     * block's first position j*r (the pages do not state the position; the
     * block start is the reading taken). */
    if (dm->idx_rope_dim > 0)
      for (int64_t j = 0; j < nbt; ++j)
        qsa_oracle_rope(pooled + j * dI, dm->idx_rope_dim, (double)dm->idx_rope_theta, j * r);
  }
  int rc = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < nq; ++i) {
    const int64_t p = pos[i], n = p + 1;
    int64_t* toks = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
    int32_t nsel = 0;
    int32_t* sl = NULL;
    if (r > 0) {
      const int64_t nb = n / r;
      float* s = (float*)malloc(sizeof(float) * (size_t)(nb > 0 ? nb : 1));
      qsa_oracle_scores(qI + i * HI * dI, w + i * HI, pooled, nb, HI, dI, c_idx, s);
      sl = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
      nsel = qsa_oracle_topk(s, nb, k, sl);
      if (scores) {
        for (int64_t j = 0; j < nb_cap; ++j)
          scores[i * nb_cap + j] = (j < nb) ? s[j] : -INFINITY;
      }
      if (sel) {
        for (int32_t t = 0; t < k; ++t) sel[i * k + t] = (t < nsel) ? sl[t] : -1;
      }
      free(s);
    }
    int64_t nt = qsa_oracle_token_set(sl, nsel, r, p, toks);
    if (n_blocks) n_blocks[i] = nsel;
    if (n_tokens) n_tokens[i] = nt;
    qsa_oracle_attend(q + i * Hq * D, K, V, gate ? gate + i * Hq * D : NULL, toks, nt, Hq, Hkv,
                      D, a_scale,
                      out + i * Hq * D);
    free(sl);
    free(toks);
  }
  free(pooled);
  return rc;
}

/* ---------------------------------------------------------------------------
 * K/V stored as 8-bit floats, optionally in a Walsh-Hadamard-rotated basis.
 *
 * "Porting Qwen4 to llama.cpp", section "Quantized KV Is a Representation
 * Contract": quantized K/V may be kept in a rotated basis H; with Q' = HQ and
 * K' = HK the scores are unchanged for orthonormal H, and a QSA attention
 * path has to honour the same storage contract as the dense path (rotate
 * before the cache write, un-rotate the output).  Here H is the Sylvester
 * Hadamard matrix of order D with entries +-1 (H H = D I), so the scores of
 * the rotated vectors carry a factor D and the output of the rotated values
 * is un-rotated as H o' / D.
 *
 * The 8-bit format is OCP E4M3 ("fn"): 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent 0 is subnormal (m * 2^-9); no
 * infinities; S.1111.111 is NaN, so the largest finite value is 448.  A
 * stored code c with scale s stands for decode(c) * s.  Encoding rounds to
 * the nearest code, ties to the even code, and saturates at +-448.
 */
float qsa_oracle_e4m3_decode(uint8_t c) {
  const int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const float v = (e == 0) ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
  return sgn ? -v : v;
}

/* Nearest finite code.  The 127 non-negative finite codes have values that
 * increase with the code, so bisection finds the first code whose value is
 * >= |x|; the nearer of it and the code below it wins, ties to the even
 * code. */
uint8_t qsa_oracle_e4m3_encode(float x) {
  if (isnan(x)) return 0x7F;
  const uint8_t sgn = signbit(x) ? 0x80 : 0x00;
  const float a = fabsf(x);
  if (a >= 448.0f) return sgn | 0x7E;
  int lo = 0, hi = 0x7E; /* decode(hi) >= a throughout */
  while (lo < hi) {
    const int mid = (lo + hi) / 2;
    if (qsa_oracle_e4m3_decode((uint8_t)mid) >= a) hi = mid;
    else lo = mid + 1;
  }
  int c = hi;
  if (c > 0) {
    const double up = (double)qsa_oracle_e4m3_decode((uint8_t)c) - (double)a;
    const double dn = (double)a - (double)qsa_oracle_e4m3_decode((uint8_t)(c - 1));
    if (dn < up || (dn == up && ((c - 1) & 1) == 0)) c = c - 1;
  }
  return sgn | (uint8_t)c;
}

/* In-place Walsh-Hadamard transform of x[0..n), n a power of two: H_n x with
 * the Sylvester H_n (entries +-1, no normalisation), in the standard order of
 * butterflies: for len = 1, 2, 4, ...: (x[j], x[j+len]) <- (x[j] + x[j+len],
 * x[j] - x[j+len]).  fp32. */
void qsa_oracle_fwht(float* x, int32_t n) {
  for (int32_t len = 1; len < n; len <<= 1)
    for (int32_t i = 0; i < n; i += 2 * len)
      for (int32_t j = i; j < i + len; ++j) {
        const float a = x[j], b = x[j + len];
        x[j] = a + b;
        x[j + len] = a - b;
      }
}

/* Storage codes of `rows` rows of D values: (rotate ? H x : x) * inv_scale,
 * encoded.  inv_scale is the fp32 reciprocal of the scale (1.0f / s). */
void qsa_oracle_kv8_encode(const float* x, int64_t rows, int32_t D, int32_t rotate,
                           float inv_scale, uint8_t* codes) {
  float* t = (float*)malloc(sizeof(float) * (size_t)D);
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t i = 0; i < D; ++i) t[i] = x[r * D + i];
    if (rotate) qsa_oracle_fwht(t, D);
    for (int32_t i = 0; i < D; ++i) codes[r * D + i] = qsa_oracle_e4m3_encode(t[i] * inv_scale);
  }
  free(t);
}

/* QSA over K/V stored as 8-bit codes (the storage above), for nq queries of
 * one sequence: as qsa_oracle_sequence, with K and V given by their codes
 * Kc, Vc [n_tok][Hkv][D] and scales.  The selection does not involve K/V.
 * With rotate, the query is rotated (q' = H q), the attention scale is
 * divided by D, and the gate-free output o' is un-rotated (H o' / D) before
 * the gate. */
int qsa_oracle_sequence_kv8(const qsa_oracle_dims* dm, int64_t n_tok, const uint8_t* Kc,
                            const uint8_t* Vc, int32_t rotate, float k_scale, float v_scale,
                            const float* kI, int64_t nq, const int64_t* pos, const float* q,
                            const float* qI, const float* w, const float* gate, float* out,
                            int32_t* sel, int32_t* n_blocks, int64_t* n_tokens, float* scores,
                            int64_t nb_cap) {
  const int32_t Hq = dm->n_q_heads, Hkv = dm->n_kv_heads, D = dm->head_dim;
  if (Hq <= 0 || Hkv <= 0 || D <= 0) return -1;
  const int64_t nkv = n_tok * Hkv * D, nqv = nq * Hq * D;
  float* Kd = (float*)malloc(sizeof(float) * (size_t)(nkv > 0 ? nkv : 1));
  float* Vd = (float*)malloc(sizeof(float) * (size_t)(nkv > 0 ? nkv : 1));
  float* qr = (float*)malloc(sizeof(float) * (size_t)(nqv > 0 ? nqv : 1));
  for (int64_t i = 0; i < nkv; ++i) {
    Kd[i] = qsa_oracle_e4m3_decode(Kc[i]) * k_scale;
    Vd[i] = qsa_oracle_e4m3_decode(Vc[i]) * v_scale;
  }
  for (int64_t i = 0; i < nqv; ++i) qr[i] = q[i];
  qsa_oracle_dims d2 = *dm;
  const double a_scale = dm->attn_scale > 0.0f ? (double)dm->attn_scale : 1.0 / sqrt((double)D);
  if (rotate) {
    for (int64_t i = 0; i < nq * Hq; ++i) qsa_oracle_fwht(qr + i * D, D);
    d2.attn_scale = (float)(a_scale / (double)D);
  }
  const int rc = qsa_oracle_sequence(&d2, n_tok, Kd, Vd, kI, nq, pos, qr, qI, w, NULL, out, sel,
                                     n_blocks, n_tokens, scores, nb_cap);
  if (rc == 0) {
    for (int64_t i = 0; i < nq * Hq; ++i) {
      float* o = out + i * D;
      if (rotate) {
        qsa_oracle_fwht(o, D);
        for (int32_t x = 0; x < D; ++x) o[x] = o[x] / (float)D;
      }
      for (int32_t x = 0; x < D; ++x) {
        const double gt = 1.0 / (1.0 + exp(-(double)gate[i * D + x]));
        o[x] = (float)((double)o[x] * gt);
      }
    }
  }
  free(Kd);
  free(Vd);
  free(qr);
  return rc;
}
