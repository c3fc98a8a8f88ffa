// Host-side GEMM wrapper (internal to the library): row-major
// C[m,n] = alpha op(A) op(B) + beta C with bf16 A and B, f32 accumulation and
// a bf16 or f32 C; op(A) is [m,k] (A stored [k,m] when trans_a), op(B) is [k,n]
// (B stored [n,k] when trans_b); lda, ldb, ldc are row strides in elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

enum class GemmStatus { kOk, kHip, kBlas };

GemmStatus gemm_bf16(bool trans_a, bool trans_b, int64_t m, int64_t n, int64_t k, float alpha, const void* A,
                     int64_t lda, const void* B, int64_t ldb, float beta, void* C, bool c_bf16, int64_t ldc,
                     hipStream_t stream);

// dst[i] = bf16(src[i]), round to nearest even
hipError_t launch_cast_bf16(int64_t n, const float* src, void* dst, hipStream_t st);

}  // namespace ssd
