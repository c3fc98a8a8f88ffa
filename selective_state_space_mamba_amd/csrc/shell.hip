// Block-shell ops around the SSD core (bandwidth-bound, no contraction):
//
//  * causal depthwise conv1d + SiLU, following depthwise_conv_preact_with_history
//    and silu on the reference page (burn_dragon_kernel src/sequence/mamba2/backward.rs):
//      preact[t,c] = bias[c] + sum_k w[c,k] xbc[t-(K-1)+k, c]   (zero before t=0)
//    and the block backward's conv/SiLU chain:
//      gp = g s (1 + p (1 - s)), s = sigmoid(p);  dbias = sum gp;
//      dw[c,k] = sum gp[t,c] xbc[t-(K-1)+k,c];   dxbc[u,c] = sum_k gp[u+K-1-k,c] w[c,k]
//  * RMSNorm-gated, following rmsnorm_gated_forward_from_inv_rms and
//    rmsnorm_gated_backward_from_inv_rms on the same page.
//
// Vector paths (taken when the x / B / C channel counts are multiples of 8, or
// the RMSNorm width is): a conv lane owns 8 (forward) or 4 (backward)
// adjacent channels and walks a run of steps (32 forward, 64 backward) with a
// register sliding window, reading 8- or 16-byte pieces of consecutive
// channels; in the backward the four waves of a workgroup take four
// consecutive runs and add their weight / bias gradient partials in LDS in
// wave order, so one partial covers 256 steps.  RMSNorm-gated takes one row per
// wave, holds the row in registers between its reduction and its outputs, and
// reduces with a wave reduction (no barrier per row).  Launch shapes are sized
// so that the block-slice workload's grids run in one round of resident waves.
// The scalar kernels (one channel per thread, a row per workgroup) take the
// other shapes.  Weight gradients are per-(batch, 256-step run) or per-64-row
// partials summed in a fixed order, so results are bitwise reproducible.
#include "gemm_launch.hpp"
#include "ssd_common.hpp"
#include "shell_launch.hpp"

namespace ssd {

constexpr int CONV_KMAX = 8;
constexpr int CONV_RUN = 256;              // steps per weight-gradient partial
constexpr int CONV_WRUN = CONV_RUN / 4;    // steps per wave in the vector backward
constexpr int CONV_FRUN = 32;              // steps per wave in the vector forward
constexpr int CONV_U = 4;                  // steps whose loads are issued together

// sigmoid with the hardware reciprocal (v_rcp_f32, 1 ulp) instead of an IEEE
// division, which costs about ten instructions per element in these
// streaming kernels; exp(-v) = inf gives 0, exp(-v) = 0 gives 1.
__device__ __forceinline__ float sigmoidf_(float v) { return __builtin_amdgcn_rcpf(1.f + __expf(-v)); }

// V (4 or 8) consecutive elements to / from floats.  f32 addresses are 16-byte
// aligned; bf16 addresses 2V-byte aligned.  bf16 stores round to nearest even.
template <int V>
__device__ __forceinline__ void ldv(const float* p, float (&f)[V]) {
#pragma unroll
  for (int i = 0; i < V; i += 4) {
    const float4 t = *reinterpret_cast<const float4*>(p + i);
    f[i] = t.x;
    f[i + 1] = t.y;
    f[i + 2] = t.z;
    f[i + 3] = t.w;
  }
}
template <int V>
__device__ __forceinline__ void ldv(const uint16_t* p, float (&f)[V]) {
  uint32_t u[V / 2];
  if constexpr (V == 8) {
    const uint4 t = *reinterpret_cast<const uint4*>(p);
    u[0] = t.x, u[1] = t.y, u[2] = t.z, u[3] = t.w;
  } else {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    u[0] = t.x, u[1] = t.y;
  }
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {
    f[2 * i] = __uint_as_float(u[i] << 16);
    f[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}
template <int V>
__device__ __forceinline__ void stv(float* p, const float (&f)[V]) {
#pragma unroll
  for (int i = 0; i < V; i += 4) *reinterpret_cast<float4*>(p + i) = make_float4(f[i], f[i + 1], f[i + 2], f[i + 3]);
}
template <int V>
__device__ __forceinline__ void stv(uint16_t* p, const float (&f)[V]) {
  if constexpr (V == 8)
    *reinterpret_cast<uint4*>(p) =
        make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7]));
  else
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]));
}
template <int V>
__device__ __forceinline__ void zerov(float (&f)[V]) {
#pragma unroll
  for (int i = 0; i < V; ++i) f[i] = 0.f;
}

// A gradient output whose dtype is chosen at run time: f32, or bf16 rounded to
// nearest even (the values a later f32 -> bf16 cast of the f32 output gives),
// and whose rows (where the kernel takes them from here) are ld elements apart.
struct GradOut {
  void* p;
  int bf;      // nonzero: bf16
  int64_t ld;  // row stride in elements
  __device__ __forceinline__ void put(int64_t i, float v) const {
    if (bf)
      static_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(v);
    else
      static_cast<float*>(p)[i] = v;
  }
  template <int V>
  __device__ __forceinline__ void putv(int64_t i, const float (&f)[V]) const {
    if (bf)
      stv<V>(static_cast<uint16_t*>(p) + i, f);
    else
      stv<V>(static_cast<float*>(p) + i, f);
  }
};

// Where channel c0 of the conv's channel axis (x, then B, then C) lives among
// the three split tensors: base pointer, row length, offset in the row.
template <typename T>
struct SplitAt {
  T* p;
  int64_t ld;
  int off;
};
template <typename T>
__device__ __forceinline__ SplitAt<T> split_at(T* x, T* B, T* C, int c0, int d_inner, int gn) {
  if (c0 < d_inner) return {x, d_inner, c0};
  if (c0 < d_inner + gn) return {B, gn, c0 - d_inner};
  return {C, gn, c0 - d_inner - gn};
}

// Taps w[c0 .. c0+V) x K (row-major [channel][tap], contiguous) into wk[k][v].
template <int V, int K>
__device__ __forceinline__ void load_taps(const float* w, int c0, float (&wk)[K][V]) {
  float raw[V * K];
#pragma unroll
  for (int i = 0; i < V * K; i += 4) {
    const float4 t = *reinterpret_cast<const float4*>(w + static_cast<int64_t>(c0) * K + i);
    raw[i] = t.x, raw[i + 1] = t.y, raw[i + 2] = t.z, raw[i + 3] = t.w;
  }
#pragma unroll
  for (int v = 0; v < V; ++v)
#pragma unroll
    for (int k = 0; k < K; ++k) wk[k][v] = raw[v * K + k];
}

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
                                                      GradOut dxbc, float* __restrict__ part, int T,
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
    dxbc.put((rb + u) * dxbc.ld + c, dsum);
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

// Vector conv forward.  grid (ceil(conv_dim / (8 * 64)), ceil(T / (4 * CONV_FRUN)), b):
// lane l owns channels c0 .. c0+7, wave q the steps [4*CONV_FRUN*y + CONV_FRUN*q, +CONV_FRUN).
template <typename TI, int K>
__global__ __launch_bounds__(256) void conv_fwd_vec_kernel(const TI* __restrict__ xbc, const float* __restrict__ w,
                                                          const float* __restrict__ bias, TI* __restrict__ x_out,
                                                          TI* __restrict__ B_out, TI* __restrict__ C_out, int T,
                                                          int Cd, int d_inner, int gn) {
  constexpr int V = 8;
  const int c0 = (blockIdx.x * WAVE + lane_id()) * V;
  const int t0 = (blockIdx.y * 4 + wave_id()) * CONV_FRUN;
  if (c0 >= Cd || t0 >= T) return;
  const int t1 = min(T, t0 + CONV_FRUN);
  const int64_t rb = static_cast<int64_t>(blockIdx.z) * T;
  float wk[K][V], bc[V];
  load_taps<V, K>(w, c0, wk);
  if (bias)
    ldv<V>(bias + c0, bc);
  else
    zerov<V>(bc);
  const SplitAt<TI> o = split_at(x_out, B_out, C_out, c0, d_inner, gn);
  // steps of loads in flight: CONV_U + 2 with bf16 activations (their window,
  // kept as the loaded words and unpacked where used, makes the room)
  constexpr int U = sizeof(TI) == 2 ? CONV_U + 2 : CONV_U;
  Vec8<TI> win[K];  // win[k] = xbc[t - (K-1) + k]
#pragma unroll
  for (int k = 0; k < K - 1; ++k) {
    const int src = t0 - (K - 1) + k;
    if (src >= 0)
      win[k].load(xbc + (rb + src) * Cd + c0);
    else
      win[k].zero();
  }
  for (int t = t0; t < t1; t += U) {
    Vec8<TI> nx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t + u < t1)
        nx[u].load(xbc + (rb + t + u) * Cd + c0);
      else
        nx[u].zero();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      win[K - 1] = nx[u];
      float a[V];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float p = bc[v];
#pragma unroll
        for (int k = 0; k < K; ++k) p += wk[k][v] * win[k].get(v);
        a[v] = p * sigmoidf_(p);
      }
      if (t + u < t1) stv<V>(o.p + (rb + t + u) * o.ld + o.off, a);
#pragma unroll
      for (int k = 0; k < K - 1; ++k) win[k] = win[k + 1];
    }
  }
}

// One step of four channels of the conv input as loaded: bf16 pairs (two
// words) or f32 (four), unpacked where used, so that the backward's window of
// 2K - 1 steps takes half the registers with bf16 activations.
template <typename TI>
struct XStep {
  float f[4];
  __device__ __forceinline__ void load(const float* p) { ldv<4>(p, f); }
  __device__ __forceinline__ void zero() { zerov<4>(f); }
  __device__ __forceinline__ float get(int v) const { return f[v]; }
};
template <>
struct XStep<uint16_t> {
  uint32_t u[2];
  __device__ __forceinline__ void load(const uint16_t* p) {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    u[0] = t.x, u[1] = t.y;
  }
  __device__ __forceinline__ void zero() { u[0] = u[1] = 0u; }
  __device__ __forceinline__ float get(int v) const {
    return (v & 1) ? __uint_as_float(u[v >> 1] & 0xFFFF0000u) : __uint_as_float(u[v >> 1] << 16);
  }
};

// Vector conv backward.  grid (ceil(conv_dim / (4 * 64)), ceil(T / CONV_RUN), b):
// lane l owns channels c0 .. c0+3, wave q the steps [CONV_RUN*y + CONV_WRUN*q, +CONV_WRUN).
// Lane state over steps u of its run:
//   xw[m] = xbc[u - (K-1) + m], m = 0 .. 2K-2   (zero outside [0, T))
//   gw[m] = gp[u + m],          m = 0 .. K-1    (zero at steps >= T)
// The workgroup's four runs add their tap / bias partials in LDS in wave order
// and store one partial [b, ceil(T/CONV_RUN), Cd, K+1] as the scalar kernel does.
// dxbc is written in TD (f32, or bf16 rounded to nearest even).
template <typename TI, int K, typename TD>
__global__ __launch_bounds__(256, K <= 4 ? 4 : 2) void conv_bwd_vec_kernel(const TI* __restrict__ xbc, const float* __restrict__ w,
                                                          const float* __restrict__ bias, const float* __restrict__ dx,
                                                          const float* __restrict__ dB, const float* __restrict__ dC,
                                                          TD* __restrict__ dxbc, int64_t ldo, float* __restrict__ part,
                                                          int T, int Cd, int d_inner, int gn) {
  // steps of loads in flight: three with bf16 activations and an f32 dxbc
  // (their packed window leaves room at 4 waves per SIMD for K = 4), two
  // otherwise (the bf16 rounding of dxbc takes that room)
  constexpr int V = 4, U = sizeof(TI) == 2 && sizeof(TD) == 4 ? 3 : 2;
  constexpr int NP = V * (K + 1);  // partial values per lane
  __shared__ float red[WAVE * NP];
  const int lane = lane_id(), wv = wave_id();
  const int cb = blockIdx.x * WAVE * V;  // first channel of the workgroup
  const int c0 = cb + lane * V;
  const int t0 = blockIdx.y * CONV_RUN + wv * CONV_WRUN;
  float acc[K + 1][V];  // taps 0..K-1, then bias
#pragma unroll
  for (int k = 0; k <= K; ++k) zerov<V>(acc[k]);
  if (c0 < Cd && t0 < T) {
    const int t1 = min(T, t0 + CONV_WRUN);
    const int64_t rb = static_cast<int64_t>(blockIdx.z) * T;
    float wk[K][V], bc[V];
    load_taps<V, K>(w, c0, wk);
    if (bias)
      ldv<V>(bias + c0, bc);
    else
      zerov<V>(bc);
    const SplitAt<const float> gi = split_at(dx, dB, dC, c0, d_inner, gn);
    auto xload = [&](int t, XStep<TI>& f) {
      if (t >= 0 && t < T)
        f.load(xbc + (rb + t) * Cd + c0);
      else
        f.zero();
    };
    auto gload = [&](int t, float (&f)[V]) {
      if (t < T)
        ldv<V>(gi.p + (rb + t) * gi.ld + gi.off, f);
      else
        zerov<V>(f);
    };
    // gp = g s (1 + p (1 - s)) for the K inputs win[0..K-1] ending at its step
    auto gp_of = [&](const float (&g)[V], const XStep<TI>* win, float (&out)[V]) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float p = bc[v];
#pragma unroll
        for (int k = 0; k < K; ++k) p += wk[k][v] * win[k].get(v);
        const float s = sigmoidf_(p);
        out[v] = g[v] * s * (1.f + p * (1.f - s));
      }
    };
    XStep<TI> xw[2 * K - 1];
    float gw[K][V];
#pragma unroll
    for (int m = 0; m < 2 * K - 1; ++m) xload(t0 - (K - 1) + m, xw[m]);
#pragma unroll
    for (int m = 0; m < K - 1; ++m) {
      float g[V];
      gload(t0 + m, g);
      gp_of(g, xw + m, gw[m]);
    }
    for (int u0 = t0; u0 < t1; u0 += U) {
      float ng[U][V];
      XStep<TI> nx[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        gload(u0 + u + K - 1, ng[u]);
        xload(u0 + u + K, nx[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (u0 + u >= t1) break;
        gp_of(ng[u], xw + (K - 1), gw[K - 1]);
        float d[V];
#pragma unroll
        for (int v = 0; v < V; ++v) {
          float sacc = 0.f;
#pragma unroll
          for (int k = 0; k < K; ++k) sacc += gw[K - 1 - k][v] * wk[k][v];
          d[v] = sacc;
        }
        stv<V>(dxbc + (rb + u0 + u) * ldo + c0, d);
#pragma unroll
        for (int v = 0; v < V; ++v) {
          acc[K][v] += gw[0][v];
#pragma unroll
          for (int k = 0; k < K; ++k) acc[k][v] += gw[0][v] * xw[k].get(v);
        }
#pragma unroll
        for (int m = 0; m < K - 1; ++m)
#pragma unroll
          for (int v = 0; v < V; ++v) gw[m][v] = gw[m + 1][v];
#pragma unroll
        for (int m = 0; m < 2 * K - 2; ++m) xw[m] = xw[m + 1];
        xw[2 * K - 2] = nx[u];
      }
    }
  }
  // The four runs' partials, added in wave order: red[(lane*V + v)*(K+1) + k].
  for (int q = 0; q < NTHREADS / WAVE; ++q) {
    if (wv == q) {
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int k = 0; k <= K; ++k) {
          float& r = red[(lane * V + v) * (K + 1) + k];
          r = q == 0 ? acc[k][v] : r + acc[k][v];
        }
    }
    __syncthreads();
  }
  const int nvalid = min(WAVE * V, Cd - cb) * (K + 1);
  float* o = part + ((static_cast<int64_t>(blockIdx.z) * gridDim.y + blockIdx.y) * Cd + cb) * (K + 1);
  for (int i = threadIdx.x; i < nvalid; i += NTHREADS) o[i] = red[i];
}

// Column sums of part [nparts, ncols] in a fixed order: wave q of a
// workgroup adds parts q, q+16, ... of 64 columns, then the 16 wave sums are
// added in wave order.  With K > 0 the columns are conv partials
// [conv_dim, K+1]: column c*(K+1)+k goes to dw[c*K+k] (k < K) or dbias[c].
constexpr int RED_WAVES = 16;
__global__ __launch_bounds__(RED_WAVES * WAVE) void part_reduce_kernel(const float* __restrict__ part,
                                                                      float* __restrict__ out,
                                                                      float* __restrict__ out_bias, int nparts,
                                                                      int64_t ncols, int K) {
  __shared__ float red[RED_WAVES][WAVE];
  const int lane = lane_id(), q = wave_id();
  const int64_t i = static_cast<int64_t>(blockIdx.x) * WAVE + lane;
  float acc = 0.f;
  if (i < ncols)
    for (int u = q; u < nparts; u += RED_WAVES) acc += part[static_cast<int64_t>(u) * ncols + i];
  red[q][lane] = acc;
  __syncthreads();
  if (q != 0 || i >= ncols) return;
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < RED_WAVES; ++k) s += red[k][lane];
  if (K == 0) {
    out[i] = s;
  } else {
    const int64_t c = i / (K + 1);
    const int k = static_cast<int>(i - c * (K + 1));
    if (k < K)
      out[c * K + k] = s;
    else
      out_bias[c] = s;
  }
}

// ------------------------------------------------------------ RMSNorm-gated

constexpr int RMS_ROWS = 64;  // rows per workgroup (one dw partial) in the backward

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
template <typename TI, typename TG, typename TO>
__global__ __launch_bounds__(256) void rms_bwd_kernel(const TI* __restrict__ y, const TI* __restrict__ z,
                                                     const float* __restrict__ w, const float* __restrict__ inv_rms,
                                                     const TG* __restrict__ g, TO* __restrict__ dy,
                                                     GradOut dz, float* __restrict__ part, int64_t rows,
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
      store_f(dy, base + i, gw * w[i] * inv - yv * coef);
      dz.put(row * dz.ld + i, gv * normalized * w[i] * s * (1.f + zv * (1.f - s)));
    }
  }
  for (int i = threadIdx.x, k = 0; i < width; i += 256, ++k) part[static_cast<int64_t>(blockIdx.x) * width + i] = dwacc[k];
}

// The loaded words of a Vec8, opaque to the compiler: values unpacked from
// them before this point are not kept live past it.
__device__ __forceinline__ void opaque_words(Vec8<uint16_t>& v) {
  asm volatile("" : "+v"(v.v.x), "+v"(v.v.y), "+v"(v.v.z), "+v"(v.v.w));
}
__device__ __forceinline__ void opaque_words(Vec8<float>& v) {
  asm volatile("" : "+v"(v.a.x), "+v"(v.a.y), "+v"(v.a.z), "+v"(v.a.w));
  asm volatile("" : "+v"(v.b.x), "+v"(v.b.y), "+v"(v.b.z), "+v"(v.b.w));
}

// Vector RMSNorm-gated: one row per wave; lane l holds the 8-element chunks
// l, l + 64, ... (KCH of them) of its row.  Needs width % 8 == 0 and
// width <= 64 * 8 * KCH.
template <typename TI, int KCH>
__global__ __launch_bounds__(256) void rms_fwd_vec_kernel(const TI* __restrict__ y, const TI* __restrict__ z,
                                                         const float* __restrict__ w, TI* __restrict__ out,
                                                         float* __restrict__ inv_rms, int64_t rows, int width,
                                                         float eps) {
  const int lane = lane_id();
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (NTHREADS / WAVE) + wave_id();
  if (row >= rows) return;
  const int nch = width / 8;
  const int64_t base = row * width;
  Vec8<TI> yr[KCH];  // the row's loaded words, unpacked where used
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < KCH; ++j) {
    const int c = lane + WAVE * j;
    if (c < nch)
      yr[j].load(y + base + 8 * c);
    else
      yr[j].zero();
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += yr[j].get(e) * yr[j].get(e);
  }
  ss = wave_sum(ss);
  // only the loaded words stay live across the reduction (see the backward)
#pragma unroll
  for (int j = 0; j < KCH; ++j) opaque_words(yr[j]);
  const float inv = 1.f / sqrtf(ss / static_cast<float>(width) + eps);
  if (lane == 0) inv_rms[row] = inv;
#pragma unroll
  for (int j = 0; j < KCH; ++j) {
    const int c = lane + WAVE * j;
    if (c >= nch) continue;
    float zv[8], wv[8], o[8];
    ldv<8>(z + base + 8 * c, zv);
    ldv<8>(w + 8 * c, wv);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = yr[j].get(e) * inv * wv[e] * zv[e] * sigmoidf_(zv[e]);
    stv<8>(out + base + 8 * c, o);
  }
}

// Vector backward: 8 waves, RMS_ROWS rows per workgroup (wave q takes rows
// q, q + 8, ...); w sits in LDS; the waves' dw partials are added in LDS in
// wave order into one partial row per workgroup.
constexpr int RMS_VEC_WAVES = 8;
template <typename TI, typename TG, typename TO, int KCH>
__global__ __launch_bounds__(RMS_VEC_WAVES * WAVE) void rms_bwd_vec_kernel(
    const TI* __restrict__ y, const TI* __restrict__ z, const float* __restrict__ w,
    const float* __restrict__ inv_rms, const TG* __restrict__ g, TO* __restrict__ dy, GradOut dz,
    float* __restrict__ part, int64_t rows, int width) {
  constexpr int NT = RMS_VEC_WAVES * WAVE;
  __shared__ float wl[8 * WAVE * KCH];
  __shared__ float red[8 * WAVE * KCH];
  const int lane = lane_id(), wq = wave_id();
  const int nch = width / 8;
  for (int i = threadIdx.x; i < width; i += NT) wl[i] = w[i];
  __syncthreads();
  float dwacc[KCH][8];
#pragma unroll
  for (int j = 0; j < KCH; ++j) zerov<8>(dwacc[j]);
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * RMS_ROWS;
  for (int i = 0; i < RMS_ROWS / RMS_VEC_WAVES; ++i) {
    const int64_t row = r0 + wq + RMS_VEC_WAVES * i;
    if (row >= rows) break;
    const int64_t base = row * width;
    const float inv = inv_rms[row];
    Vec8<TI> yr[KCH], zr[KCH];
    Vec8<TG> gr[KCH];
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int c = lane + WAVE * j;
      if (c < nch) {
        yr[j].load(y + base + 8 * c);
        zr[j].load(z + base + 8 * c);
        gr[j].load(g + base + 8 * c);
      } else {
        yr[j].zero(), zr[j].zero(), gr[j].zero();
      }
    }
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int c = lane + WAVE * j;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float zv = zr[j].get(e);
        const float wv = c < nch ? wl[8 * c + e] : 0.f;
        dot += gr[j].get(e) * zv * sigmoidf_(zv) * wv * yr[j].get(e);
      }
    }
    dot = wave_sum(dot);
    const float coef = dot * inv * inv * inv / static_cast<float>(width);
    // Only the loaded words stay live across the reduction: the outputs
    // recompute sigmoid(z) and the unpacked values from them.
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      opaque_words(yr[j]);
      opaque_words(zr[j]);
      opaque_words(gr[j]);
    }
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int c = lane + WAVE * j;
      if (c >= nch) continue;
      float o_dy[8], o_dz[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float zv = zr[j].get(e), yv = yr[j].get(e), gv = gr[j].get(e), wv = wl[8 * c + e];
        const float s = sigmoidf_(zv);
        const float gate = zv * s, normalized = yv * inv;
        const float gwv = gv * gate;
        dwacc[j][e] += gwv * normalized;
        o_dy[e] = gwv * wv * inv - yv * coef;
        o_dz[e] = gv * normalized * wv * s * (1.f + zv * (1.f - s));
      }
      stv<8>(dy + base + 8 * c, o_dy);
      dz.putv<8>(row * dz.ld + 8 * c, o_dz);
    }
  }
  for (int q = 0; q < RMS_VEC_WAVES; ++q) {
    if (wq == q) {
#pragma unroll
      for (int j = 0; j < KCH; ++j) {
        const int c = lane + WAVE * j;
        if (c >= nch) continue;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float& r = red[8 * c + e];
          r = q == 0 ? dwacc[j][e] : r + dwacc[j][e];
        }
      }
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < width; i += NT) part[static_cast<int64_t>(blockIdx.x) * width + i] = red[i];
}

// ------------------------------------------------------------ dt activation
//
// dt = softplus(dt_raw + dt_bias[h]) with beta 1, and its backward
// ddt_raw = ddt * sigmoid(dt_raw + dt_bias[h]), d_dt_bias[h] = sum over rows of
// ddt_raw, following the dt_pre / softplus lines of tensorized_mamba2_backward_impl
// and the grad_dt_pre / grad_dt_bias lines after the fused backward on the page
// (burn_dragon_kernel src/sequence/mamba2/backward.rs).  softplus(v) = log(1 + e^v) is
// evaluated as max(v, 0) + log1p(e^-|v|), the same function without overflow.
// Rows are the b*T steps of a [b, T, H] array.

constexpr int DT_ROWS = 64;  // rows per workgroup (one d_dt_bias partial) in the backward

__device__ __forceinline__ float softplus1(float v) { return fmaxf(v, 0.f) + log1pf(expf(-fabsf(v))); }

template <typename T>
__global__ __launch_bounds__(256) void dt_softplus_fwd_kernel(const T* __restrict__ raw,
                                                             const float* __restrict__ bias, T* __restrict__ dt,
                                                             int64_t n, int H) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  store_f(dt, i, softplus1(load_f(raw, i) + bias[i % H]));
}

// grid ceil(rows / DT_ROWS), 256 threads: thread t takes head h = hb + t % hpb
// and rows r0 + t / hpb + k * (256 / hpb); the row lanes of a head are added in
// LDS in lane order.  part: [gridDim.x, H].
template <typename T>
__global__ __launch_bounds__(256) void dt_softplus_bwd_kernel(const T* __restrict__ raw,
                                                             const float* __restrict__ bias,
                                                             const float* __restrict__ ddt, GradOut ddt_raw,
                                                             float* __restrict__ part, int64_t rows, int H) {
  __shared__ float red[256];
  const int tid = threadIdx.x;
  const int hpb = H < 256 ? H : 256;  // heads per pass
  const int S = 256 / hpb;            // row lanes per head
  const int hi = tid % hpb, s = tid / hpb;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * DT_ROWS;
  const int64_t r1 = r0 + DT_ROWS < rows ? r0 + DT_ROWS : rows;
  for (int hb = 0; hb < H; hb += hpb) {
    const int h = hb + hi;
    float acc = 0.f;
    if (s < S && h < H) {
      const float bh = bias[h];
#pragma unroll 4
      for (int64_t r = r0 + s; r < r1; r += S) {
        const int64_t i = r * H + h;
        const float g = ddt[i] / (1.f + expf(-(load_f(raw, i) + bh)));
        ddt_raw.put(r * ddt_raw.ld + h, g);
        acc += g;
      }
    }
    red[tid] = acc;
    __syncthreads();
    if (tid < hpb && hb + tid < H) {
      float sum = 0.f;
      for (int q = 0; q < S; ++q) sum += red[q * hpb + tid];
      part[static_cast<int64_t>(blockIdx.x) * H + hb + tid] = sum;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- launchers

int conv_nruns(int T) { return (T + CONV_RUN - 1) / CONV_RUN; }
int rms_nparts(int64_t rows) { return static_cast<int>((rows + RMS_ROWS - 1) / RMS_ROWS); }
int rms_max_width() { return 256 * 16; }
int conv_max_k() { return CONV_KMAX; }

// The vector conv paths need every 8-channel piece inside one of x, B, C.
static bool conv_vec_ok(int d_inner, int gn) { return d_inner % 8 == 0 && gn % 8 == 0; }

template <typename TI, int K>
static void conv_fwd_launch(int b, int T, int Cd, int d_inner, int gn, const void* xbc, const float* w,
                            const float* bias, void* x_out, void* B_out, void* C_out, hipStream_t st) {
  if (conv_vec_ok(d_inner, gn)) {
    dim3 grid((Cd / 8 + WAVE - 1) / WAVE, (T + 4 * CONV_FRUN - 1) / (4 * CONV_FRUN), b);
    hipLaunchKernelGGL((conv_fwd_vec_kernel<TI, K>), grid, dim3(NTHREADS), 0, st, static_cast<const TI*>(xbc), w,
                       bias, static_cast<TI*>(x_out), static_cast<TI*>(B_out), static_cast<TI*>(C_out), T, Cd, d_inner,
                       gn);
  } else {
    dim3 grid((Cd + 255) / 256, conv_nruns(T), b);
    hipLaunchKernelGGL((conv_fwd_kernel<TI, K>), grid, dim3(256), 0, st, static_cast<const TI*>(xbc), w, bias,
                       static_cast<TI*>(x_out), static_cast<TI*>(B_out), static_cast<TI*>(C_out), T, Cd, d_inner, gn,
                       CONV_RUN);
  }
}

template <typename TI, int K>
static void conv_bwd_launch(int b, int T, int Cd, int d_inner, int gn, const void* xbc, const float* w,
                            const float* bias, const float* dx, const float* dB, const float* dC, GradOut dxbc,
                            float* part, hipStream_t st) {
  if (conv_vec_ok(d_inner, gn)) {
    dim3 grid((Cd / 4 + WAVE - 1) / WAVE, conv_nruns(T), b);
    if (dxbc.bf)
      hipLaunchKernelGGL((conv_bwd_vec_kernel<TI, K, uint16_t>), grid, dim3(NTHREADS), 0, st,
                         static_cast<const TI*>(xbc), w, bias, dx, dB, dC, static_cast<uint16_t*>(dxbc.p), dxbc.ld,
                         part, T, Cd, d_inner, gn);
    else
      hipLaunchKernelGGL((conv_bwd_vec_kernel<TI, K, float>), grid, dim3(NTHREADS), 0, st,
                         static_cast<const TI*>(xbc), w, bias, dx, dB, dC, static_cast<float*>(dxbc.p), dxbc.ld,
                         part, T, Cd, d_inner, gn);
  } else {
    dim3 grid((Cd + 255) / 256, conv_nruns(T), b);
    hipLaunchKernelGGL((conv_bwd_kernel<TI, K>), grid, dim3(256), 0, st, static_cast<const TI*>(xbc), w, bias, dx,
                       dB, dC, dxbc, part, T, Cd, d_inner, gn, CONV_RUN);
  }
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

static void launch_part_reduce(const float* part, float* out, float* out_bias, int nparts, int64_t ncols, int K,
                               hipStream_t st) {
  hipLaunchKernelGGL(part_reduce_kernel, dim3(static_cast<unsigned>((ncols + WAVE - 1) / WAVE)),
                     dim3(RED_WAVES * WAVE), 0, st, part, out, out_bias, nparts, ncols, K);
}

hipError_t launch_conv_fwd(int b, int T, int d_inner, int gn, int K, DType dt, const void* xbc, const float* w,
                           const float* bias, void* x_out, void* B_out, void* C_out, hipStream_t st) {
  const int Cd = d_inner + 2 * gn;
  if (dt == BF16) {
    SSD_CONV_DISPATCH(conv_fwd_launch, uint16_t, b, T, Cd, d_inner, gn, xbc, w, bias, x_out, B_out, C_out, st)
  } else {
    SSD_CONV_DISPATCH(conv_fwd_launch, float, b, T, Cd, d_inner, gn, xbc, w, bias, x_out, B_out, C_out, st)
  }
  return hipGetLastError();
}

hipError_t launch_conv_bwd(int b, int T, int d_inner, int gn, int K, DType dt, const void* xbc, const float* w,
                           const float* bias, const float* dx, const float* dB, const float* dC, void* dxbc,
                           DType dxt, int64_t dxbc_ld, float* dw, float* dbias, float* part, hipStream_t st) {
  const int Cd = d_inner + 2 * gn;
  const GradOut go{dxbc, dxt == BF16 ? 1 : 0, dxbc_ld};
  if (dt == BF16) {
    SSD_CONV_DISPATCH(conv_bwd_launch, uint16_t, b, T, Cd, d_inner, gn, xbc, w, bias, dx, dB, dC, go, part, st)
  } else {
    SSD_CONV_DISPATCH(conv_bwd_launch, float, b, T, Cd, d_inner, gn, xbc, w, bias, dx, dB, dC, go, part, st)
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_part_reduce(part, dw, dbias, b * conv_nruns(T), static_cast<int64_t>(Cd) * (K + 1), K, st);
  return hipGetLastError();
}

// Chunks of 8 per lane the vector RMSNorm kernels are instantiated for.
static int rms_kch(int width) {
  const int need = (width / 8 + WAVE - 1) / WAVE;
  return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 6 ? 6 : 8;
}

template <typename TI>
static void rms_fwd_launch(int64_t rows, int width, float eps, const void* y, const void* z, const float* w,
                           void* out, float* inv_rms, hipStream_t st) {
  const TI* yp = static_cast<const TI*>(y);
  const TI* zp = static_cast<const TI*>(z);
  TI* op = static_cast<TI*>(out);
  if (width % 8 != 0) {
    hipLaunchKernelGGL(rms_fwd_kernel<TI>, dim3(rows), dim3(256), 0, st, yp, zp, w, op, inv_rms, width, eps);
    return;
  }
  const dim3 grid(static_cast<unsigned>((rows + NTHREADS / WAVE - 1) / (NTHREADS / WAVE)));
  switch (rms_kch(width)) {
    case 1: hipLaunchKernelGGL((rms_fwd_vec_kernel<TI, 1>), grid, dim3(NTHREADS), 0, st, yp, zp, w, op, inv_rms, rows, width, eps); break;
    case 2: hipLaunchKernelGGL((rms_fwd_vec_kernel<TI, 2>), grid, dim3(NTHREADS), 0, st, yp, zp, w, op, inv_rms, rows, width, eps); break;
    case 4: hipLaunchKernelGGL((rms_fwd_vec_kernel<TI, 4>), grid, dim3(NTHREADS), 0, st, yp, zp, w, op, inv_rms, rows, width, eps); break;
    case 6: hipLaunchKernelGGL((rms_fwd_vec_kernel<TI, 6>), grid, dim3(NTHREADS), 0, st, yp, zp, w, op, inv_rms, rows, width, eps); break;
    default: hipLaunchKernelGGL((rms_fwd_vec_kernel<TI, 8>), grid, dim3(NTHREADS), 0, st, yp, zp, w, op, inv_rms, rows, width, eps); break;
  }
}

hipError_t launch_rms_fwd(int64_t rows, int width, float eps, DType dt, const void* y, const void* z, const float* w,
                          void* out, float* inv_rms, hipStream_t st) {
  if (dt == BF16)
    rms_fwd_launch<uint16_t>(rows, width, eps, y, z, w, out, inv_rms, st);
  else
    rms_fwd_launch<float>(rows, width, eps, y, z, w, out, inv_rms, st);
  return hipGetLastError();
}

template <typename TI, typename TG, typename TO>
static void rms_bwd_launch(int64_t rows, int width, const void* y, const void* z, const float* w,
                           const float* inv_rms, const void* g, void* dy, GradOut dz, float* part, hipStream_t st) {
  const TI* yp = static_cast<const TI*>(y);
  const TI* zp = static_cast<const TI*>(z);
  const TG* gp = static_cast<const TG*>(g);
  TO* dyp = static_cast<TO*>(dy);
  const dim3 grid(rms_nparts(rows));
  // The vector kernel holds up to 6 chunks of 8 per lane (width <= 3072) of
  // three operands in registers; all-f32 operands fit up to 4 chunks.
  const int kch = rms_kch(width);
  const bool vec = width % 8 == 0 && (kch <= 4 || (kch == 6 && (sizeof(TI) == 2 || sizeof(TG) == 2)));
  if (!vec) {
    hipLaunchKernelGGL((rms_bwd_kernel<TI, TG, TO>), grid, dim3(256), 0, st, yp, zp, w, inv_rms, gp, dyp, dz, part,
                       rows, width);
    return;
  }
  const dim3 block(RMS_VEC_WAVES * WAVE);
  switch (kch) {
    case 1: hipLaunchKernelGGL((rms_bwd_vec_kernel<TI, TG, TO, 1>), grid, block, 0, st, yp, zp, w, inv_rms, gp, dyp, dz, part, rows, width); break;
    case 2: hipLaunchKernelGGL((rms_bwd_vec_kernel<TI, TG, TO, 2>), grid, block, 0, st, yp, zp, w, inv_rms, gp, dyp, dz, part, rows, width); break;
    case 4: hipLaunchKernelGGL((rms_bwd_vec_kernel<TI, TG, TO, 4>), grid, block, 0, st, yp, zp, w, inv_rms, gp, dyp, dz, part, rows, width); break;
    default:
      if constexpr (sizeof(TI) == 2 || sizeof(TG) == 2)
        hipLaunchKernelGGL((rms_bwd_vec_kernel<TI, TG, TO, 6>), grid, block, 0, st, yp, zp, w, inv_rms, gp, dyp, dz, part, rows, width);
      break;
  }
}

template <typename TI, typename TG>
static void rms_bwd_launch_o(DType ot, int64_t rows, int width, const void* y, const void* z, const float* w,
                             const float* inv_rms, const void* g, void* dy, GradOut dz, float* part, hipStream_t st) {
  if (ot == BF16)
    rms_bwd_launch<TI, TG, uint16_t>(rows, width, y, z, w, inv_rms, g, dy, dz, part, st);
  else
    rms_bwd_launch<TI, TG, float>(rows, width, y, z, w, inv_rms, g, dy, dz, part, st);
}

hipError_t launch_rms_bwd(int64_t rows, int width, DType dt, DType gt, DType ot, const void* y, const void* z,
                          const float* w, const float* inv_rms, const void* g, void* dy, void* dz, DType zt,
                          int64_t dz_ld, float* dw, float* part, hipStream_t st) {
  const GradOut go{dz, zt == BF16 ? 1 : 0, dz_ld};
  if (dt == BF16) {
    if (gt == BF16)
      rms_bwd_launch_o<uint16_t, uint16_t>(ot, rows, width, y, z, w, inv_rms, g, dy, go, part, st);
    else
      rms_bwd_launch_o<uint16_t, float>(ot, rows, width, y, z, w, inv_rms, g, dy, go, part, st);
  } else {
    if (gt == BF16)
      rms_bwd_launch_o<float, uint16_t>(ot, rows, width, y, z, w, inv_rms, g, dy, go, part, st);
    else
      rms_bwd_launch_o<float, float>(ot, rows, width, y, z, w, inv_rms, g, dy, go, part, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_part_reduce(part, dw, nullptr, rms_nparts(rows), width, 0, st);
  return hipGetLastError();
}

int dt_nparts(int64_t rows) { return static_cast<int>((rows + DT_ROWS - 1) / DT_ROWS); }

hipError_t launch_dt_softplus_fwd(int64_t rows, int H, DType dt, const void* raw, const float* bias, void* out,
                                  hipStream_t st) {
  const int64_t n = rows * H;
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  if (dt == BF16)
    hipLaunchKernelGGL(dt_softplus_fwd_kernel<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(raw),
                       bias, static_cast<uint16_t*>(out), n, H);
  else
    hipLaunchKernelGGL(dt_softplus_fwd_kernel<float>, grid, dim3(256), 0, st, static_cast<const float*>(raw), bias,
                       static_cast<float*>(out), n, H);
  return hipGetLastError();
}

hipError_t launch_dt_softplus_bwd(int64_t rows, int H, DType dt, const void* raw, const float* bias, const float* ddt,
                                  void* ddt_raw, DType ot, int64_t ld, float* d_bias, float* part, hipStream_t st) {
  const dim3 grid(dt_nparts(rows));
  const GradOut go{ddt_raw, ot == BF16 ? 1 : 0, ld};
  if (dt == BF16)
    hipLaunchKernelGGL(dt_softplus_bwd_kernel<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(raw),
                       bias, ddt, go, part, rows, H);
  else
    hipLaunchKernelGGL(dt_softplus_bwd_kernel<float>, grid, dim3(256), 0, st, static_cast<const float*>(raw), bias,
                       ddt, go, part, rows, H);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_part_reduce(part, d_bias, nullptr, dt_nparts(rows), H, 0, st);
  return hipGetLastError();
}

// f32 -> bf16 (round to nearest even), four elements per thread when aligned.
__global__ __launch_bounds__(256) void cast_bf16_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst,
                                                       int64_t n) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i + 4 <= n) {
    float f[4];
    ldv<4>(src + i, f);
    stv<4>(dst + i, f);
  } else {
    for (int64_t e = i; e < n; ++e) dst[e] = f32_to_bf16_bits(src[e]);
  }
}

hipError_t launch_cast_bf16(int64_t n, const float* src, void* dst, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 1023) / 1024;
  hipLaunchKernelGGL(cast_bf16_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, src,
                     static_cast<uint16_t*>(dst), n);
  return hipGetLastError();
}

}  // namespace ssd
