// Chunk output of the SSD forward.
//
// Inside one chunk (s_i = within-chunk inclusive cumsum of dt A, H_c the state
// entering the chunk) the recurrence of the page-1 reference
// (burn_dragon_kernel mamba2/backward.rs, ssd_forward_state_history_reference,
// with the y readout of the block backward: y = sum_n ssm C + D x) is
//
//   y_i = sum_{j<=i} exp(s_i - s_j) (C_i . B_j) dt_j x_j     (intra-chunk part)
//       + exp(s_i) C_i . H_c^T                                (incoming state)
//       + D x_i.
//
// A workgroup owns one 64-row block ib of chunk c for a run of heads of one
// group.  It computes the group's C.B^T tiles (ib, jb <= ib) once with MFMA
// (K = d_state) and keeps them in registers, then per head applies the decay
// mask L_ij = exp(s_i - s_j) (i >= j; exponents are <= 0) and dt_j, and runs
// the two remaining contractions (K = chunk block, K = d_state) on MFMA.
#include "ssd_common.hpp"
#include "ssd_launch.hpp"

namespace ssd {

template <typename TI, bool BF>
__global__ __launch_bounds__(NTHREADS) void chunk_out_fwd_kernel(
    const TI* __restrict__ x, const TI* __restrict__ Bm, const TI* __restrict__ Cm,
    const TI* __restrict__ dt, const float* __restrict__ A_log, const float* __restrict__ D,
    const float* __restrict__ hstates, TI* __restrict__ y, int T, int H, int P, int N, int G, int Q,
    int nsplit) {
  typedef typename Op<BF>::T OT;
  constexpr int PAD = BF ? 8 : 4;
  constexpr int LDN = NMAX + PAD;  // [row][n]
  constexpr int LDQ = BQ + PAD;    // [row][j] and [p][j]
  __shared__ __attribute__((aligned(16))) OT sC[BQ * LDN];
  __shared__ __attribute__((aligned(16))) OT sBH[BQ * LDN];  // B block, then H_c as [p][n]
  __shared__ __attribute__((aligned(16))) OT sXt[PMAX * LDQ];
  __shared__ __attribute__((aligned(16))) OT sG[BQ * LDQ];
  __shared__ float sS[QMAX];
  __shared__ float sDt[QMAX];
  __shared__ float sTmp[8];

  const int nc = T / Q, nb = (Q + BQ - 1) / BQ;
  const int hpg = H / G, hps = hpg / nsplit;
  int idx = blockIdx.x;
  const int ib = idx % nb;
  idx /= nb;
  const int sp = idx % nsplit;
  idx /= nsplit;
  const int g = idx % G;
  idx /= G;
  const int c = idx % nc;
  const int bi = idx / nc;

  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), r = l & 15, q = l >> 4;
  const int64_t t0 = static_cast<int64_t>(c) * Q;
  const int i0 = ib * BQ;
  const int vi = min(BQ, Q - i0);
  const int Kn = round_up(N, Op<BF>::KS);
  const int64_t GN = static_cast<int64_t>(G) * N, HP = static_cast<int64_t>(H) * P;

  // ---- group-level C.B^T tiles for (ib, jb <= ib)
  stage_tile<TI, OT, false>(sC, LDN, Cm + ((static_cast<int64_t>(bi) * T + t0 + i0) * G + g) * N, GN, BQ,
                            NMAX, vi, N);
  f4 cb[NBMAX][4];
#pragma unroll
  for (int jb = 0; jb < NBMAX; ++jb) {
    zero(cb[jb]);
    if (jb <= ib) {
      __syncthreads();
      stage_tile<TI, OT, false>(sBH, LDN, Bm + ((static_cast<int64_t>(bi) * T + t0 + jb * BQ) * G + g) * N,
                                GN, BQ, NMAX, min(BQ, Q - jb * BQ), N);
      __syncthreads();
      wave_gemm<BF, true, true, 4>(cb[jb], sC + 16 * w * LDN, LDN, 1, sBH, LDN, 1, Kn);
    }
  }

  for (int hh = 0; hh < hps; ++hh) {
    const int h = g * hpg + sp * hps + hh;
    const float A = -__expf(A_log[h]);
    const float Dh = D[h];
    __syncthreads();
    const float dtv = (tid < Q) ? load_f(dt, (static_cast<int64_t>(bi) * T + t0 + tid) * H + h) : 0.f;
    const float s = block_inclusive_scan(dtv * A, sTmp);
    if (tid < Q) {
      sS[tid] = s;
      sDt[tid] = dtv;
    }
    stage_tile<float, OT, false>(sBH, LDN,
                                 hstates + ((static_cast<int64_t>(bi) * nc + c) * H + h) * static_cast<int64_t>(P) * N,
                                 N, PMAX, NMAX, P, N);
    __syncthreads();

    // incoming-state readout: exp(s_i) * C_i . H_c^T
    f4 acc[4];
    zero(acc);
    wave_gemm<BF, true, true, 4>(acc, sC + 16 * w * LDN, LDN, 1, sBH, LDN, 1, Kn);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int iq = i0 + 16 * w + 4 * q + i;
      const float e = (iq < Q) ? __expf(sS[iq]) : 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t][i] *= e;
    }

    // intra-chunk part, one 64-column block of the chunk at a time
#pragma unroll
    for (int jb = 0; jb < NBMAX; ++jb) {
      if (jb <= ib) {
        __syncthreads();
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int il = 16 * w + 4 * q + i;
            const int iq = i0 + il, jq = jb * BQ + 16 * ct + r;
            float v = 0.f;
            if (iq < Q && jq <= iq) v = cb[jb][ct][i] * __expf(sS[iq] - sS[jq]) * sDt[jq];
            sG[il * LDQ + 16 * ct + r] = Op<BF>::cvt(v);
          }
        stage_tile<TI, OT, true>(sXt, LDQ, x + ((static_cast<int64_t>(bi) * T + t0 + jb * BQ) * H + h) * P, HP,
                                 BQ, PMAX, min(BQ, Q - jb * BQ), P);
        __syncthreads();
        wave_gemm<BF, true, true, 4>(acc, sG + 16 * w * LDQ, LDQ, 1, sXt, LDQ, 1, BQ);
      }
    }

    // skip term and store
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int iq = i0 + 16 * w + 4 * q + i, p = 16 * t + r;
        if (iq < Q && p < P) {
          const int64_t o = ((static_cast<int64_t>(bi) * T + t0 + iq) * H + h) * P + p;
          store_f(y, o, acc[t][i] + Dh * load_f(x, o));
        }
      }
  }
}

hipError_t launch_chunk_out_fwd(const Dims& d, DType act, int nsplit, const void* x, const void* B,
                                const void* C, const void* dt, const float* A_log, const float* D,
                                const float* states, void* y, hipStream_t st) {
  const int64_t nblk = static_cast<int64_t>(d.b) * d.nc() * d.G * nsplit * d.nb();
  if (act == BF16) {
    hipLaunchKernelGGL((chunk_out_fwd_kernel<uint16_t, true>), dim3(nblk), dim3(NTHREADS), 0, st,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(B),
                       static_cast<const uint16_t*>(C), static_cast<const uint16_t*>(dt), A_log, D, states,
                       static_cast<uint16_t*>(y), d.T, d.H, d.P, d.N, d.G, d.Q, nsplit);
  } else {
    hipLaunchKernelGGL((chunk_out_fwd_kernel<float, false>), dim3(nblk), dim3(NTHREADS), 0, st,
                       static_cast<const float*>(x), static_cast<const float*>(B),
                       static_cast<const float*>(C), static_cast<const float*>(dt), A_log, D, states,
                       static_cast<float*>(y), d.T, d.H, d.P, d.N, d.G, d.Q, nsplit);
  }
  return hipGetLastError();
}

}  // namespace ssd
