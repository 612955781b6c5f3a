// The block front end's prefill-sized projections as plain library GEMMs on
// hipBLASLt: D[M][N] = A[M][K] · B[N][K]ᵀ, bf16 inputs, fp32 accumulation,
// fp32 or bf16 output, both row-major (a Linear layer's activations and
// weight).  hipBLASLt is opened with dlopen on the first such product, so
// nothing loads it before a GPU call needs it; when it is missing, has no
// algorithm for the shape, or the stream is being captured before the shape
// has a plan (creating one allocates), the caller runs its own tiled kernel.
#include <dlfcn.h>
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <atomic>
#include <map>
#include <mutex>
#include <tuple>

#include "qsa_internal.h"

namespace qsa {
namespace {

// The entry points used, looked up by name (the C API).
struct LtApi {
  decltype(&hipblasLtCreate) create = nullptr;
  decltype(&hipblasLtMatmulDescCreate) desc_create = nullptr;
  decltype(&hipblasLtMatmulDescDestroy) desc_destroy = nullptr;
  decltype(&hipblasLtMatrixLayoutDestroy) layout_destroy = nullptr;
  decltype(&hipblasLtMatmulDescSetAttribute) desc_set = nullptr;
  decltype(&hipblasLtMatrixLayoutCreate) layout_create = nullptr;
  decltype(&hipblasLtMatmulPreferenceCreate) pref_create = nullptr;
  decltype(&hipblasLtMatmulPreferenceSetAttribute) pref_set = nullptr;
  decltype(&hipblasLtMatmulPreferenceDestroy) pref_destroy = nullptr;
  decltype(&hipblasLtMatmulAlgoGetHeuristic) heuristic = nullptr;
  decltype(&hipblasLtMatmul) matmul = nullptr;
};

struct LtPlan {
  bool ok = false;
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasLtMatmulAlgo_t algo{};
};

struct LtDevice {
  bool tried = false;
  hipblasLtHandle_t h = nullptr;
  std::map<std::tuple<int, int, int, int>, LtPlan> plans;  // (M, N, K, fp32 out)
};

constexpr int kMaxDevices = 64;
// Plans kept per device (one per product shape; the token count varies from
// call to call): past this many the cache is emptied and rebuilt on demand.
// The heuristic picks the same algorithm for a shape every time, so the
// kernel a shape runs does not depend on the calls before it.
constexpr size_t kMaxPlans = 64;
#ifdef QSA_COUNT_KEYS
std::atomic<bool> g_off{false};  // (debug builds) hipBLASLt switched off by a test
#endif
std::mutex g_mu;
bool g_api_tried = false;
LtApi g_api;
LtDevice g_dev[kMaxDevices];

bool load_api() {
  if (g_api_tried) return g_api.matmul != nullptr;
  g_api_tried = true;
  void* so = dlopen("libhipblaslt.so.1", RTLD_NOW | RTLD_LOCAL);
  if (so == nullptr) so = dlopen("libhipblaslt.so", RTLD_NOW | RTLD_LOCAL);
  if (so == nullptr) return false;
  LtApi a;
  a.create = reinterpret_cast<decltype(a.create)>(dlsym(so, "hipblasLtCreate"));
  a.desc_create = reinterpret_cast<decltype(a.desc_create)>(dlsym(so, "hipblasLtMatmulDescCreate"));
  a.desc_destroy = reinterpret_cast<decltype(a.desc_destroy)>(dlsym(so, "hipblasLtMatmulDescDestroy"));
  a.layout_destroy = reinterpret_cast<decltype(a.layout_destroy)>(dlsym(so, "hipblasLtMatrixLayoutDestroy"));
  a.desc_set = reinterpret_cast<decltype(a.desc_set)>(dlsym(so, "hipblasLtMatmulDescSetAttribute"));
  a.layout_create = reinterpret_cast<decltype(a.layout_create)>(dlsym(so, "hipblasLtMatrixLayoutCreate"));
  a.pref_create = reinterpret_cast<decltype(a.pref_create)>(dlsym(so, "hipblasLtMatmulPreferenceCreate"));
  a.pref_set = reinterpret_cast<decltype(a.pref_set)>(dlsym(so, "hipblasLtMatmulPreferenceSetAttribute"));
  a.pref_destroy = reinterpret_cast<decltype(a.pref_destroy)>(dlsym(so, "hipblasLtMatmulPreferenceDestroy"));
  a.heuristic = reinterpret_cast<decltype(a.heuristic)>(dlsym(so, "hipblasLtMatmulAlgoGetHeuristic"));
  a.matmul = reinterpret_cast<decltype(a.matmul)>(dlsym(so, "hipblasLtMatmul"));
  if (!a.create || !a.desc_create || !a.desc_destroy || !a.desc_set || !a.layout_create ||
      !a.layout_destroy || !a.pref_create || !a.pref_set || !a.pref_destroy || !a.heuristic ||
      !a.matmul)
    return false;
  g_api = a;
  return true;
}

// In hipBLASLt's column-major terms the row-major product is Dᵀ (N x M) =
// op(B') · A', with B' the weight seen as a K x N matrix (transposed by the
// operation) and A' the activations as K x M; no workspace.
LtPlan make_plan(hipblasLtHandle_t h, int M, int N, int K, bool d_f32) {
  const LtApi& a = g_api;
  LtPlan p;
  bool ok = a.desc_create(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
  const hipblasOperation_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
  ok = ok && a.desc_set(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT)) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && a.desc_set(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN)) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && a.layout_create(&p.la, HIP_R_16BF, K, N, K) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && a.layout_create(&p.lb, HIP_R_16BF, K, M, K) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && a.layout_create(&p.ld, d_f32 ? HIP_R_32F : HIP_R_16BF, N, M, N) == HIPBLAS_STATUS_SUCCESS;
  hipblasLtMatmulPreference_t pref = nullptr;
  ok = ok && a.pref_create(&pref) == HIPBLAS_STATUS_SUCCESS;
  const uint64_t ws = 0;
  ok = ok && a.pref_set(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws, sizeof(ws)) ==
                 HIPBLAS_STATUS_SUCCESS;
  hipblasLtMatmulHeuristicResult_t res[1];
  int n = 0;
  ok = ok && a.heuristic(h, p.desc, p.la, p.lb, p.ld, p.ld, pref, 1, res, &n) == HIPBLAS_STATUS_SUCCESS;
  if (pref != nullptr) a.pref_destroy(pref);
  p.ok = ok && n > 0 && res[0].state == HIPBLAS_STATUS_SUCCESS && res[0].workspaceSize == 0;
  if (p.ok) p.algo = res[0].algo;
  return p;
}

void free_plans(LtDevice& L) {
  for (auto& kv : L.plans) {
    LtPlan& p = kv.second;
    if (p.la != nullptr) g_api.layout_destroy(p.la);
    if (p.lb != nullptr) g_api.layout_destroy(p.lb);
    if (p.ld != nullptr) g_api.layout_destroy(p.ld);
    if (p.desc != nullptr) g_api.desc_destroy(p.desc);
  }
  L.plans.clear();
}

}  // namespace

#ifdef QSA_COUNT_KEYS
void lt_set_enabled(bool on) { g_off = !on; }
#endif

hipError_t lt_gemm(const void* A, const void* B, void* D, bool d_f32, int M, int N, int K,
                   hipStream_t st) {
#ifdef QSA_COUNT_KEYS
  if (g_off) return hipErrorNotSupported;
#endif
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return hipErrorNotSupported;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cap) != hipSuccess) return hipErrorNotSupported;
  std::lock_guard<std::mutex> lock(g_mu);
  LtDevice& L = g_dev[dev];
  const auto key = std::make_tuple(M, N, K, d_f32 ? 1 : 0);
  auto it = L.plans.find(key);
  if (it == L.plans.end()) {
    if (cap != hipStreamCaptureStatusNone) return hipErrorNotSupported;  // setup allocates
    if (!load_api()) return hipErrorNotSupported;
    if (!L.tried) {
      L.tried = true;
      if (g_api.create(&L.h) != HIPBLAS_STATUS_SUCCESS) L.h = nullptr;
    }
    if (L.h == nullptr) return hipErrorNotSupported;
    if (L.plans.size() >= kMaxPlans) free_plans(L);
    it = L.plans.emplace(key, make_plan(L.h, M, N, K, d_f32)).first;
  }
  const LtPlan& p = it->second;
  if (!p.ok) return hipErrorNotSupported;
  const float alpha = 1.0f, beta = 0.0f;
  const hipblasStatus_t s = g_api.matmul(L.h, p.desc, &alpha, B, p.la, A, p.lb, &beta, D, p.ld, D,
                                         p.ld, &p.algo, nullptr, 0, st);
  return s == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorLaunchFailure;
}

}  // namespace qsa
