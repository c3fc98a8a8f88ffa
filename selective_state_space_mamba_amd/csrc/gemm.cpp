// Plain GEMMs for the projections around the SSD block slice (bf16 operands,
// f32 accumulation, bf16 or f32 result).  The row-major product
// C = alpha op(A) op(B) + beta C is the column-major product
// C^T = op(B)^T op(A)^T, so the operands are handed to the library swapped.
//
// hipBLASLt by default: per device one handle and one workspace, created on
// first use, and per problem shape the descriptors and an algorithm, kept for
// the later calls of that shape.  The algorithm is the fastest of the (up to
// 32) candidates the library's heuristic offers, timed on the shape's first
// call into a scratch output (so that an accumulating call, beta != 0, does
// not see the trial runs); that first call synchronises its stream.  rocBLAS
// (gemm_ex) takes the shapes for which hipBLASLt offers no algorithm, and all
// of them under SSD_GEMM=rocblas.  Calls are serialised under one lock (the
// handles' streams are set per call).
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>
#include <rocblas/rocblas.h>

#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "gemm_launch.hpp"

namespace ssd {

namespace {
std::mutex g_blas_mu;
std::map<int, rocblas_handle> g_blas;

constexpr size_t kLtWorkspace = size_t(128) << 20;  // bytes of hipBLASLt workspace per device

struct LtDevice {
  hipblasLtHandle_t handle = nullptr;
  void* workspace = nullptr;
};
std::map<int, LtDevice> g_lt;

// One problem shape: its descriptors and the chosen algorithm (ok = false:
// hipBLASLt offered none, rocBLAS takes it).
struct LtPlan {
  bool ok = false;
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo;
  size_t ws = 0;
};
typedef std::tuple<int, bool, bool, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, bool> LtKey;
std::map<LtKey, LtPlan> g_lt_plans;

bool use_hipblaslt() {
  static const bool lt = [] {
    const char* v = std::getenv("SSD_GEMM");
    return !(v && std::strcmp(v, "rocblas") == 0);
  }();
  return lt;
}

GemmStatus rocblas_gemm(int dev, bool trans_a, bool trans_b, int64_t m, int64_t n, int64_t k, float alpha,
                        const void* A, int64_t lda, const void* B, int64_t ldb, float beta, void* C, bool c_bf16,
                        int64_t ldc, hipStream_t stream) {
  rocblas_handle& h = g_blas[dev];
  if (!h && rocblas_create_handle(&h) != rocblas_status_success) {
    h = nullptr;
    return GemmStatus::kBlas;
  }
  if (rocblas_set_stream(h, stream) != rocblas_status_success) return GemmStatus::kBlas;
  const rocblas_datatype ct = c_bf16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
  const rocblas_status st = rocblas_gemm_ex_64(
      h, trans_b ? rocblas_operation_transpose : rocblas_operation_none,
      trans_a ? rocblas_operation_transpose : rocblas_operation_none, n, m, k, &alpha, B, rocblas_datatype_bf16_r,
      ldb, A, rocblas_datatype_bf16_r, lda, &beta, C, ct, ldc, C, ct, ldc, rocblas_datatype_f32_r,
      rocblas_gemm_algo_standard, 0, 0);
  return st == rocblas_status_success ? GemmStatus::kOk : GemmStatus::kBlas;
}

constexpr int kLtCandidates = 32;

// Mean time in ms of `reps` runs of one algorithm (negative if it fails).
float lt_time(LtDevice& d, const LtPlan& p, const hipblasLtMatmulAlgo_t& algo, size_t ws, const void* A,
              const void* B, float alpha, float beta, void* Cs, hipStream_t stream, int reps) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess) return -1.f;
  if (hipEventCreate(&e1) != hipSuccess) {
    hipEventDestroy(e0);
    return -1.f;
  }
  float ms = -1.f;
  bool ok = hipblasLtMatmul(d.handle, p.desc, &alpha, B, p.la, A, p.lb, &beta, Cs, p.lc, Cs, p.lc, &algo,
                            d.workspace, ws, stream) == HIPBLAS_STATUS_SUCCESS;  // warm-up
  ok = ok && hipEventRecord(e0, stream) == hipSuccess;
  for (int r = 0; ok && r < reps; ++r)
    ok = hipblasLtMatmul(d.handle, p.desc, &alpha, B, p.la, A, p.lb, &beta, Cs, p.lc, Cs, p.lc, &algo,
                         d.workspace, ws, stream) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipEventRecord(e1, stream) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
       hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  return ok ? ms / reps : -1.f;
}

// The plan of one shape, made on its first call (see the head of the file).
const LtPlan* lt_plan(int dev, LtDevice& d, bool trans_a, bool trans_b, int64_t m, int64_t n, int64_t k,
                      int64_t lda, int64_t ldb, int64_t ldc, bool c_bf16, const void* A, const void* B, float alpha,
                      float beta, hipStream_t stream) {
  const LtKey key{dev, trans_a, trans_b, m, n, k, lda, ldb, ldc, c_bf16};
  auto it = g_lt_plans.find(key);
  if (it != g_lt_plans.end()) return &it->second;
  LtPlan& p = g_lt_plans[key];
  // column-major: "A" is B^T-side operand [n x k] (op N) or [k x n] (op T),
  // "B" is the A-side operand [k x m] (op N) or [m x k] (op T), C is [n x m]
  const hipblasOperation_t opa = trans_b ? HIPBLAS_OP_T : HIPBLAS_OP_N;
  const hipblasOperation_t opb = trans_a ? HIPBLAS_OP_T : HIPBLAS_OP_N;
  const hipDataType ct = c_bf16 ? HIP_R_16BF : HIP_R_32F;
  bool ok = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opa, sizeof(opa)) ==
                 HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opb, sizeof(opb)) ==
                 HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, trans_b ? k : n, trans_b ? n : k, ldb) ==
                 HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, trans_a ? m : k, trans_a ? k : m, lda) ==
                 HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&p.lc, ct, n, m, ldc) == HIPBLAS_STATUS_SUCCESS;
  if (ok) {
    hipblasLtMatmulPreference_t pref = nullptr;
    const uint64_t wsmax = kLtWorkspace;
    hipblasLtMatmulHeuristicResult_t res[kLtCandidates];
    int nres = 0;
    ok = hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsmax,
                                               sizeof(wsmax)) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulAlgoGetHeuristic(d.handle, p.desc, p.la, p.lb, p.lc, p.lc, pref, kLtCandidates, res,
                                         &nres) == HIPBLAS_STATUS_SUCCESS;
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    int best = -1;
    float best_ms = 0.f;
    void* Cs = nullptr;  // scratch output for the trials (its contents do not matter to their time)
    const size_t cbytes = (static_cast<size_t>(m - 1) * ldc + n) * (c_bf16 ? 2 : 4);
    const bool trials = ok && nres > 1 && hipMalloc(&Cs, cbytes) == hipSuccess;
    for (int i = 0; ok && i < nres; ++i) {
      if (res[i].state != HIPBLAS_STATUS_SUCCESS || res[i].workspaceSize > kLtWorkspace) continue;
      if (!trials) {  // one candidate (or no scratch): the first usable one
        best = i;
        break;
      }
      const float ms = lt_time(d, p, res[i].algo, res[i].workspaceSize, A, B, alpha, beta, Cs, stream, 3);
      if (ms >= 0.f && (best < 0 || ms < best_ms)) best = i, best_ms = ms;
    }
    if (Cs) {
      hipStreamSynchronize(stream);
      hipFree(Cs);
    }
    ok = ok && best >= 0;
    if (ok) {
      p.algo = res[best].algo;
      p.ws = res[best].workspaceSize;
    }
  }
  p.ok = ok;
  return &p;
}
}  // namespace

GemmStatus gemm_bf16(bool trans_a, bool trans_b, int64_t m, int64_t n, int64_t k, float alpha, const void* A,
                     int64_t lda, const void* B, int64_t ldb, float beta, void* C, bool c_bf16, int64_t ldc,
                     hipStream_t stream) {
  std::lock_guard<std::mutex> lk(g_blas_mu);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GemmStatus::kHip;
  if (use_hipblaslt()) {
    LtDevice& d = g_lt[dev];
    if (!d.handle) {
      if (hipblasLtCreate(&d.handle) != HIPBLAS_STATUS_SUCCESS) {
        d.handle = nullptr;
        return GemmStatus::kBlas;
      }
      if (hipMalloc(&d.workspace, kLtWorkspace) != hipSuccess) {
        d.workspace = nullptr;
        return GemmStatus::kHip;
      }
    }
    const LtPlan* p = lt_plan(dev, d, trans_a, trans_b, m, n, k, lda, ldb, ldc, c_bf16, A, B, alpha, beta, stream);
    if (p->ok) {
      const hipblasStatus_t st = hipblasLtMatmul(d.handle, p->desc, &alpha, B, p->la, A, p->lb, &beta, C, p->lc, C,
                                                 p->lc, &p->algo, d.workspace, p->ws, stream);
      return st == HIPBLAS_STATUS_SUCCESS ? GemmStatus::kOk : GemmStatus::kBlas;
    }
  }
  return rocblas_gemm(dev, trans_a, trans_b, m, n, k, alpha, A, lda, B, ldb, beta, C, c_bf16, ldc, stream);
}

}  // namespace ssd
