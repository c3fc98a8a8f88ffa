// Host-side launchers of the block-shell kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_launch.hpp"

namespace ssd {

int conv_nruns(int T);
int rms_nparts(int64_t rows);
int rms_max_width();
int conv_max_k();

hipError_t launch_conv_fwd(int b, int T, int d_inner, int gn, int K, DType dt, const void* xbc, const float* w,
                           const float* bias, void* x_out, void* B_out, void* C_out, hipStream_t st);
// part: [b * conv_nruns(T), conv_dim, K + 1] floats of scratch; dxbc in `dxt`
// (f32 or bf16), its b*T rows dxbc_ld elements apart
hipError_t launch_conv_bwd(int b, int T, int d_inner, int gn, int K, DType dt, const void* xbc, const float* w,
                           const float* bias, const float* dx, const float* dB, const float* dC, void* dxbc,
                           DType dxt, int64_t dxbc_ld, float* dw, float* dbias, float* part, hipStream_t st);
hipError_t launch_rms_fwd(int64_t rows, int width, float eps, DType dt, const void* y, const void* z, const float* w,
                          void* out, float* inv_rms, hipStream_t st);
// part: [rms_nparts(rows), width] floats of scratch
// dy in `ot`, dz in `zt` (f32 or bf16), dz's rows dz_ld elements apart; dw f32
hipError_t launch_rms_bwd(int64_t rows, int width, DType dt, DType gt, DType ot, const void* y, const void* z,
                          const float* w, const float* inv_rms, const void* g, void* dy, void* dz, DType zt,
                          int64_t dz_ld, float* dw, float* part, hipStream_t st);

// dt = softplus(raw + bias[h]) over rows x H, in `dt` (f32 or bf16)
int dt_nparts(int64_t rows);
hipError_t launch_dt_softplus_fwd(int64_t rows, int H, DType dt, const void* raw, const float* bias, void* out,
                                  hipStream_t st);
// part: [dt_nparts(rows), H] floats of scratch; ddt_raw in `ot` (f32 or bf16),
// its rows ld elements apart
hipError_t launch_dt_softplus_bwd(int64_t rows, int H, DType dt, const void* raw, const float* bias, const float* ddt,
                                  void* ddt_raw, DType ot, int64_t ld, float* d_bias, float* part, hipStream_t st);

}  // namespace ssd
