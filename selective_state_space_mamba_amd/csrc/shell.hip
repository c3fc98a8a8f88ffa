// Block-shell ops around the SSD core (bandwidth-bound, no contraction):
//
//  * causal depthwise conv1d + SiLU, following depthwise_conv_preact_with_history
//    and silu on the page-1 reference (burn_dragon_kernel mamba2/backward.rs):
//      preact[t,c] = bias[c] + sum_k w[c,k] xbc[t-(K-1)+k, c]   (zero before t=0)
//    and the block backward's conv/SiLU chain:
//      gp = g s (1 + p (1 - s)), s = sigmoid(p);  dbias = sum gp;
//      dw[c,k] = sum gp[t,c] xbc[t-(K-1)+k,c];   dxbc[u,c] = sum_k gp[u+K-1-k,c] w[c,k]
//  * RMSNorm-gated, following rmsnorm_gated_forward_from_inv_rms and
//    rmsnorm_gated_backward_from_inv_rms on the same page.
//
// Conv threads own one channel and walk a run of time steps with a register
// sliding window (reads coalesced across channels); weight/bias gradients are
// written as per-(batch, time-run) partials and summed in a fixed order.
#include "ssd_common.hpp"
#include "shell_launch.hpp"

namespace ssd {

constexpr int CONV_KMAX = 8;

__device__ __forceinline__ float sigmoidf_(float v) { return 1.f / (1.f + __expf(-v)); }

template <typename TI>
__device__ __forceinline__ void store_split(TI* x_out, TI* B_out, TI* C_out, int64_t row, int c, int d_inner,
                                            int gn, float v) {
  if (c < d_inner)
    store_f(x_out, row * d_inner + c, v);
  else if (c < d_inner + gn)
    store_f(B_out, row * gn + (c - d_inner), v);
  else
    store_f(C_out, row * gn + (c - d_inner - gn), v);
}

template <typename TI, int K>
__global__ __launch_bounds__(256) void conv_fwd_kernel(const TI* __restrict__ xbc, const float* __restrict__ w,
                                                      const float* __restrict__ bias, TI* __restrict__ x_out,
                                                      TI* __restrict__ B_out, TI* __restrict__ C_out, int T, int Cd,
                                                      int d_inner, int gn, int run) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= Cd) return;
  const int bi = blockIdx.z;
  const int t0 = blockIdx.y * run, t1 = min(T, t0 + run);
  const int64_t rb = static_cast<int64_t>(bi) * T;
  float wk[K], win[K];
#pragma unroll
  for (int k = 0; k < K; ++k) wk[k] = w[c * K + k];
  const float bc = bias ? bias[c] : 0.f;
  // win[k] = xbc[t - (K-1) + k]
#pragma unroll
  for (int k = 0; k < K - 1; ++k) {
    const int src = t0 - (K - 1) + k;
    win[k] = src >= 0 ? load_f(xbc, (rb + src) * Cd + c) : 0.f;
  }
  for (int t = t0; t < t1; ++t) {
    win[K - 1] = load_f(xbc, (rb + t) * Cd + c);
    float p = bc;
#pragma unroll
    for (int k = 0; k < K; ++k) p += wk[k] * win[k];
    store_split(x_out, B_out, C_out, rb + t, c, d_inner, gn, p * sigmoidf_(p));
#pragma unroll
    for (int k = 0; k < K - 1; ++k) win[k] = win[k + 1];
  }
}

__device__ __forceinline__ float gact_at(const float* dx, const float* dB, const float* dC, int64_t row, int c,
                                         int d_inner, int gn) {
  if (c < d_inner) return dx[row * d_inner + c];
  if (c < d_inner + gn) return dB[row * gn + (c - d_inner)];
  return dC[row * gn + (c - d_inner - gn)];
}

// One thread per channel walks steps u in [t0, t1) keeping
//   xw[m] = xbc[u - (K-1) + m], m = 0 .. 2K-2   (zero outside [0, T))
//   gw[m] = gp[u + m],          m = 0 .. K-1    (zero at steps >= T)
// partials: [b, nruns, Cd, K+1] (K weight taps, then bias)
template <typename TI, int K>
__global__ __launch_bounds__(256) void conv_bwd_kernel(const TI* __restrict__ xbc, const float* __restrict__ w,
                                                      const float* __restrict__ bias, const float* __restrict__ dx,
                                                      const float* __restrict__ dB, const float* __restrict__ dC,
                                                      float* __restrict__ dxbc, float* __restrict__ part, int T,
                                                      int Cd, int d_inner, int gn, int run) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= Cd) return;
  const int bi = blockIdx.z, nruns = gridDim.y;
  const int t0 = blockIdx.y * run, t1 = min(T, t0 + run);
  const int64_t rb = static_cast<int64_t>(bi) * T;
  float wk[K], xw[2 * K - 1], gw[K], acc[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    wk[k] = w[c * K + k];
    acc[k] = 0.f;
  }
  const float bc = bias ? bias[c] : 0.f;
  float accb = 0.f;
  auto xat = [&](int t) -> float { return (t >= 0 && t < T) ? load_f(xbc, (rb + t) * Cd + c) : 0.f; };
  // gp at step t from the K inputs ending at t (win[0..K-1] = xbc[t-(K-1) .. t])
  auto gp_at = [&](int t, const float* win) -> float {
    if (t >= T) return 0.f;
    float p = bc;
#pragma unroll
    for (int k = 0; k < K; ++k) p += wk[k] * win[k];
    const float s = sigmoidf_(p);
    return gact_at(dx, dB, dC, rb + t, c, d_inner, gn) * s * (1.f + p * (1.f - s));
  };
#pragma unroll
  for (int m = 0; m < 2 * K - 1; ++m) xw[m] = xat(t0 - (K - 1) + m);
#pragma unroll
  for (int m = 0; m < K - 1; ++m) gw[m] = gp_at(t0 + m, xw + m);
  for (int u = t0; u < t1; ++u) {
    gw[K - 1] = gp_at(u + K - 1, xw + (K - 1));
    float dsum = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) dsum += gw[K - 1 - k] * wk[k];
    dxbc[(rb + u) * Cd + c] = dsum;
    accb += gw[0];
#pragma unroll
    for (int k = 0; k < K; ++k) acc[k] += gw[0] * xw[k];
#pragma unroll
    for (int m = 0; m < K - 1; ++m) gw[m] = gw[m + 1];
#pragma unroll
    for (int m = 0; m < 2 * K - 2; ++m) xw[m] = xw[m + 1];
    xw[2 * K - 2] = xat(u + K);
  }
  float* o = part + ((static_cast<int64_t>(bi) * nruns + blockIdx.y) * Cd + c) * (K + 1);
#pragma unroll
  for (int k = 0; k < K; ++k) o[k] = acc[k];
  o[K] = accb;
}

__global__ __launch_bounds__(256) void conv_param_reduce_kernel(const float* __restrict__ part,
                                                               float* __restrict__ dw, float* __restrict__ dbias,
                                                               int nparts, int Cd, int K) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= Cd) return;
  float acc[CONV_KMAX + 1];
  for (int k = 0; k <= K; ++k) acc[k] = 0.f;
  for (int u = 0; u < nparts; ++u)
    for (int k = 0; k <= K; ++k) acc[k] += part[(static_cast<int64_t>(u) * Cd + c) * (K + 1) + k];
  for (int k = 0; k < K; ++k) dw[c * K + k] = acc[k];
  dbias[c] = acc[K];
}

// ------------------------------------------------------------ RMSNorm-gated

constexpr int RMS_ROWS = 32;  // rows per workgroup in the backward

__device__ __forceinline__ float block_sum256(float v, float* tmp) {
  v = wave_sum(v);
  __syncthreads();
  if (lane_id() == 0) tmp[wave_id()] = v;
  __syncthreads();
  return tmp[0] + tmp[1] + tmp[2] + tmp[3];
}

template <typename TI>
__global__ __launch_bounds__(256) void rms_fwd_kernel(const TI* __restrict__ y, const TI* __restrict__ z,
                                                     const float* __restrict__ w, TI* __restrict__ out,
                                                     float* __restrict__ inv_rms, int width, float eps) {
  __shared__ float tmp[4];
  const int64_t row = blockIdx.x;
  const int64_t base = row * width;
  float ss = 0.f;
  for (int i = threadIdx.x; i < width; i += 256) {
    const float v = load_f(y, base + i);
    ss += v * v;
  }
  ss = block_sum256(ss, tmp);
  const float inv = 1.f / sqrtf(ss / static_cast<float>(width) + eps);
  if (threadIdx.x == 0) inv_rms[row] = inv;
  for (int i = threadIdx.x; i < width; i += 256) {
    const float zv = load_f(z, base + i);
    store_f(out, base + i, load_f(y, base + i) * inv * w[i] * zv * sigmoidf_(zv));
  }
}

// dw partials: [ceil(rows/RMS_ROWS), width]
template <typename TI, typename TG>
__global__ __launch_bounds__(256) void rms_bwd_kernel(const TI* __restrict__ y, const TI* __restrict__ z,
                                                     const float* __restrict__ w, const float* __restrict__ inv_rms,
                                                     const TG* __restrict__ g, float* __restrict__ dy,
                                                     float* __restrict__ dz, float* __restrict__ part, int64_t rows,
                                                     int width) {
  __shared__ float tmp[4];
  constexpr int MAXPER = 16;  // width <= 256 * MAXPER
  float dwacc[MAXPER];
  for (int k = 0; k < MAXPER; ++k) dwacc[k] = 0.f;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * RMS_ROWS;
  const int64_t r1 = r0 + RMS_ROWS < rows ? r0 + RMS_ROWS : rows;
  for (int64_t row = r0; row < r1; ++row) {
    const int64_t base = row * width;
    const float inv = inv_rms[row];
    float dot = 0.f;
    for (int i = threadIdx.x, k = 0; i < width; i += 256, ++k) {
      const float zv = load_f(z, base + i);
      dot += load_f(g, base + i) * zv * sigmoidf_(zv) * w[i] * load_f(y, base + i);
    }
    dot = block_sum256(dot, tmp);
    const float coef = dot * inv * inv * inv / static_cast<float>(width);
    for (int i = threadIdx.x, k = 0; i < width; i += 256, ++k) {
      const float zv = load_f(z, base + i), yv = load_f(y, base + i), gv = load_f(g, base + i);
      const float s = sigmoidf_(zv);
      const float gate = zv * s, normalized = yv * inv;
      const float gw = gv * gate;
      dwacc[k] += gw * normalized;
      dy[base + i] = gw * w[i] * inv - yv * coef;
      dz[base + i] = gv * normalized * w[i] * s * (1.f + zv * (1.f - s));
    }
  }
  for (int i = threadIdx.x, k = 0; i < width; i += 256, ++k) part[static_cast<int64_t>(blockIdx.x) * width + i] = dwacc[k];
}

__global__ __launch_bounds__(256) void rms_param_reduce_kernel(const float* __restrict__ part, float* __restrict__ dw,
                                                              int nparts, int width) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= width) return;
  float acc = 0.f;
  for (int u = 0; u < nparts; ++u) acc += part[static_cast<int64_t>(u) * width + i];
  dw[i] = acc;
}

// ---------------------------------------------------------------- launchers

constexpr int CONV_RUN = 128;

int conv_nruns(int T) { return (T + CONV_RUN - 1) / CONV_RUN; }
int rms_nparts(int64_t rows) { return static_cast<int>((rows + RMS_ROWS - 1) / RMS_ROWS); }
int rms_max_width() { return 256 * 16; }
int conv_max_k() { return CONV_KMAX; }

template <typename TI, int K>
static void conv_fwd_launch(dim3 grid, int T, int Cd, int d_inner, int gn, const void* xbc, const float* w,
                            const float* bias, void* x_out, void* B_out, void* C_out, hipStream_t st) {
  hipLaunchKernelGGL((conv_fwd_kernel<TI, K>), grid, dim3(256), 0, st, static_cast<const TI*>(xbc), w, bias,
                     static_cast<TI*>(x_out), static_cast<TI*>(B_out), static_cast<TI*>(C_out), T, Cd, d_inner, gn,
                     CONV_RUN);
}

template <typename TI, int K>
static void conv_bwd_launch(dim3 grid, int T, int Cd, int d_inner, int gn, const void* xbc, const float* w,
                            const float* bias, const float* dx, const float* dB, const float* dC, float* dxbc,
                            float* part, hipStream_t st) {
  hipLaunchKernelGGL((conv_bwd_kernel<TI, K>), grid, dim3(256), 0, st, static_cast<const TI*>(xbc), w, bias, dx, dB,
                     dC, dxbc, part, T, Cd, d_inner, gn, CONV_RUN);
}

#define SSD_CONV_DISPATCH(FN, TI, ...)      \
  switch (K) {                              \
    case 1: FN<TI, 1>(__VA_ARGS__); break;  \
    case 2: FN<TI, 2>(__VA_ARGS__); break;  \
    case 3: FN<TI, 3>(__VA_ARGS__); break;  \
    case 4: FN<TI, 4>(__VA_ARGS__); break;  \
    case 5: FN<TI, 5>(__VA_ARGS__); break;  \
    case 6: FN<TI, 6>(__VA_ARGS__); break;  \
    case 7: FN<TI, 7>(__VA_ARGS__); break;  \
    default: FN<TI, 8>(__VA_ARGS__); break; \
  }

hipError_t launch_conv_fwd(int b, int T, int d_inner, int gn, int K, DType dt, const void* xbc, const float* w,
                           const float* bias, void* x_out, void* B_out, void* C_out, hipStream_t st) {
  const int Cd = d_inner + 2 * gn;
  dim3 grid((Cd + 255) / 256, conv_nruns(T), b);
  if (dt == BF16) {
    SSD_CONV_DISPATCH(conv_fwd_launch, uint16_t, grid, T, Cd, d_inner, gn, xbc, w, bias, x_out, B_out, C_out, st)
  } else {
    SSD_CONV_DISPATCH(conv_fwd_launch, float, grid, T, Cd, d_inner, gn, xbc, w, bias, x_out, B_out, C_out, st)
  }
  return hipGetLastError();
}

hipError_t launch_conv_bwd(int b, int T, int d_inner, int gn, int K, DType dt, const void* xbc, const float* w,
                           const float* bias, const float* dx, const float* dB, const float* dC, float* dxbc,
                           float* dw, float* dbias, float* part, hipStream_t st) {
  const int Cd = d_inner + 2 * gn;
  dim3 grid((Cd + 255) / 256, conv_nruns(T), b);
  if (dt == BF16) {
    SSD_CONV_DISPATCH(conv_bwd_launch, uint16_t, grid, T, Cd, d_inner, gn, xbc, w, bias, dx, dB, dC, dxbc, part, st)
  } else {
    SSD_CONV_DISPATCH(conv_bwd_launch, float, grid, T, Cd, d_inner, gn, xbc, w, bias, dx, dB, dC, dxbc, part, st)
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(conv_param_reduce_kernel, dim3((Cd + 255) / 256), dim3(256), 0, st, part, dw, dbias,
                     b * conv_nruns(T), Cd, K);
  return hipGetLastError();
}

hipError_t launch_rms_fwd(int64_t rows, int width, float eps, DType dt, const void* y, const void* z, const float* w,
                          void* out, float* inv_rms, hipStream_t st) {
  if (dt == BF16)
    hipLaunchKernelGGL(rms_fwd_kernel<uint16_t>, dim3(rows), dim3(256), 0, st, static_cast<const uint16_t*>(y),
                       static_cast<const uint16_t*>(z), w, static_cast<uint16_t*>(out), inv_rms, width, eps);
  else
    hipLaunchKernelGGL(rms_fwd_kernel<float>, dim3(rows), dim3(256), 0, st, static_cast<const float*>(y),
                       static_cast<const float*>(z), w, static_cast<float*>(out), inv_rms, width, eps);
  return hipGetLastError();
}

template <typename TI, typename TG>
static void rms_bwd_launch(int64_t rows, int width, const void* y, const void* z, const float* w,
                           const float* inv_rms, const void* g, float* dy, float* dz, float* part, hipStream_t st) {
  hipLaunchKernelGGL((rms_bwd_kernel<TI, TG>), dim3(rms_nparts(rows)), dim3(256), 0, st, static_cast<const TI*>(y),
                     static_cast<const TI*>(z), w, inv_rms, static_cast<const TG*>(g), dy, dz, part, rows, width);
}

hipError_t launch_rms_bwd(int64_t rows, int width, DType dt, DType gt, const void* y, const void* z, const float* w,
                          const float* inv_rms, const void* g, float* dy, float* dz, float* dw, float* part,
                          hipStream_t st) {
  if (dt == BF16) {
    if (gt == BF16)
      rms_bwd_launch<uint16_t, uint16_t>(rows, width, y, z, w, inv_rms, g, dy, dz, part, st);
    else
      rms_bwd_launch<uint16_t, float>(rows, width, y, z, w, inv_rms, g, dy, dz, part, st);
  } else {
    if (gt == BF16)
      rms_bwd_launch<float, uint16_t>(rows, width, y, z, w, inv_rms, g, dy, dz, part, st);
    else
      rms_bwd_launch<float, float>(rows, width, y, z, w, inv_rms, g, dy, dz, part, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rms_param_reduce_kernel, dim3((width + 255) / 256), dim3(256), 0, st, part, dw, rms_nparts(rows),
                     width);
  return hipGetLastError();
}

}  // namespace ssd
