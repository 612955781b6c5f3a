/* Test probe of the QSA library: present only in the debug build
 * libqsa_probe.so (compiled with QSA_COUNT_KEYS), never in libqsa.so.
 *
 * The gather, not a mask (llama.cpp PR #27739 page, LocalAI QSA-block
 * commit, section "What the context length buys": the block reads
 * keys_visited = n_sel rows per query and KV head, not the dense prefix):
 * every attention kernel of the probe build adds the number of valid K/V
 * rows it loads to one device counter.  After a call, the counter equals the
 * sum over the call's (query token, KV head) units of the token set size
 * r * min(k, nb) + tail (every visible row for a dense layer). */
#ifndef QSA_PROBE_H
#define QSA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The counter's value (after all work on the device has finished: the read
 * is a synchronous copy); reset != 0 sets it to zero afterwards.  -1 on a
 * HIP error. */
int64_t qsa_probe_keys_visited(int32_t reset);

/* The block front end's prefill-sized projections run on hipBLASLt where it
 * is present; enable = 0 makes them run the library's own LDS-tiled MFMA
 * kernel instead (until called again with a non-zero value), so that tests
 * cover both.  Process-wide; not thread-safe against running calls. */
void qsa_probe_library_gemm(int32_t enable);

/* One product D[M][N] = A[M][K] B[N][K]^T (bf16 inputs, row-major; D fp32
 * when d_f32, else bf16) through the library's hipBLASLt path, enqueued on
 * `stream` (a hipStream_t; NULL = the null stream).  Device pointers.
 * Returns 0 when enqueued, 1 when hipBLASLt cannot run it (missing, no
 * algorithm, or stream capture before the shape has a plan), -1 on bad
 * arguments or a failed launch. */
int32_t qsa_probe_gemm(const void* A, const void* B, void* D, int32_t d_f32, int32_t M, int32_t N,
                       int32_t K, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_PROBE_H */
