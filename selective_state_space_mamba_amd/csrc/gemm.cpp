// Plain GEMMs for the projections around the SSD block slice, through rocBLAS
// (gemm_ex: bf16 operands, f32 accumulation, bf16 or f32 result).  The row-
// major product C = alpha op(A) op(B) + beta C is the column-major product
// C^T = op(B)^T op(A)^T, so the operands are handed to rocBLAS swapped.  One
// rocBLAS handle per device, created on first use; its stream is set for each
// call under a lock, so calls from several threads are ordered on the handle.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <map>
#include <mutex>

#include "gemm_launch.hpp"

namespace ssd {

namespace {
std::mutex g_blas_mu;
std::map<int, rocblas_handle> g_blas;
}  // namespace

GemmStatus gemm_bf16(bool trans_a, bool trans_b, int64_t m, int64_t n, int64_t k, float alpha, const void* A,
                     int64_t lda, const void* B, int64_t ldb, float beta, void* C, bool c_bf16, int64_t ldc,
                     hipStream_t stream) {
  std::lock_guard<std::mutex> lk(g_blas_mu);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GemmStatus::kHip;
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

}  // namespace ssd
