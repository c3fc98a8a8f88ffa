// Intra-chunk backward of the SSD and the dt / A / D reductions.
//
// Gradients of L = sum(dy * y) for one chunk follow from the reverse-time loop
// of the page-1 reference (burn_dragon_kernel mamba2/backward.rs,
// ssd_backward_reference) regrouped by chunk.  Notation: s_i within-chunk
// inclusive cumsum of dt A, L_ij = exp(s_i - s_j) for i >= j, CB_ij = C_i . B_j,
// yx_ij = dy_i . x_j, H_c the state entering the chunk, Gamma the gradient
// reaching the state that leaves it (from the state-gradient pass),
// V_j = x_j Gamma (a d_state vector), U_i = dy_i H_c.
//
//   dx_j = D dy_j + dt_j [ sum_{i>=j} L_ij CB_ij dy_i + exp(s_end - s_j) B_j Gamma^T ]
//   dB_j = sum_{heads of the group} dt_j [ sum_{i>=j} L_ij yx_ij C_i + exp(s_end - s_j) V_j ]
//   dC_i = sum_{heads of the group} [ sum_{j<=i} L_ij yx_ij dt_j B_j + exp(s_i) U_i ]
//
// The decay enters through s; with E_ij = L_ij CB_ij yx_ij and M_ij = E_ij dt_j,
//   ds_k = sum_{j<k} M_kj - sum_{i>k} M_ik + exp(s_k) U_k . C_k - R_k
//          + [k = last] ( sum_j R_j + exp(s_end) <Gamma, H_c> ),
//   R_j = dt_j exp(s_end - s_j) V_j . B_j,
// da_t = sum_{k>=t} ds_k, and the reference's two dt terms become
//   ddt_t = sum_{i>=t} E_it + R_t / dt_t + A da_t,
//   dA_log = A sum_{b,t} dt_t da_t,   dD = sum dy . x.
//
// Two MFMA kernels split the work by output orientation:
//  * column kernel: one 64-row block jb of a chunk, all i-blocks >= jb: dx_j,
//    dB_j, column sums of E, diagonal of E, R_j / dt_j.
//  * row kernel: one 64-row block ib, all j-blocks <= ib: dC_i, row sums of M,
//    the readout term exp(s_i) U_i . C_i, and dD partials.
// Both loop over the heads of one group (or a run of them) so the group's
// C.B^T tiles are computed once, and they sum the head-dependent matrices
// L yx dt over heads before the single contraction with C (or B) that dB (dC)
// needs.  Every cross-workgroup sum goes through fixed-order partial buffers
// (no atomics), so results are bitwise reproducible.
#include <type_traits>

#include "ssd_common.hpp"
#include "ssd_launch.hpp"

namespace ssd {

// Sum over the workgroup; result valid in every thread.  `tmp`: 4 floats.
__device__ __forceinline__ float block_sum(float v, float* tmp) {
  v = wave_sum(v);
  __syncthreads();
  if (lane_id() == 0) tmp[wave_id()] = v;
  __syncthreads();
  return tmp[0] + tmp[1] + tmp[2] + tmp[3];
}

// Chunk rows (or columns) staged per slab: the whole chunk for bf16 operands,
// 64 at a time for f32.
template <bool BF> struct BwdSlab { static constexpr int W = BF ? QMAX : BQ; };

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// ------------------------------------------------------------ column kernel

template <typename TI, typename TY, bool BF>
__global__ __launch_bounds__(NTHREADS) void chunk_bwd_col_kernel(
    const TI* __restrict__ x, const TI* __restrict__ Bm, const TI* __restrict__ Cm,
    const TI* __restrict__ dt, const TY* __restrict__ dy, const float* __restrict__ A_log,
    const float* __restrict__ D, const typename Op<BF>::T* __restrict__ gamma, float* __restrict__ dx,
    float* __restrict__ dB_out, float* __restrict__ colE, float* __restrict__ diagE,
    float* __restrict__ Rp, int T, int H, int P, int N, int G, int Q, int nsplit) {
  typedef typename Op<BF>::T OT;
  constexpr int PAD = BF ? 8 : 4;
  constexpr int IW = BwdSlab<BF>::W;
  constexpr int LDN = NMAX + PAD, LDP = PMAX + PAD, LDI = IW + PAD;
  constexpr int R_PH1 = IW * LDN;                                       // C rows [i][n]
  constexpr int R_DIAG = IW * LDP + (BF ? PMAX * LDI : 0) + BQ * LDI;   // dy [i][p], dy^T [p][i], G1^T [j][i]
  constexpr int R_STATE = PMAX * LDN + (BF ? NMAX * LDP : 0);           // Gamma [p][n], Gamma^T [n][p]
  constexpr int R_FIN = BQ * LDI + (BF ? NMAX * LDI : IW * LDN);        // W^T [j][i], C^T [n][i] or C [i][n]
  constexpr int RSZ = cmax(cmax(R_PH1, R_DIAG), cmax(R_STATE, R_FIN));
  __shared__ __attribute__((aligned(16))) OT sB[BQ * LDN];  // B_jb [j][n]
  __shared__ __attribute__((aligned(16))) OT sX[BQ * LDP];  // x_jb [j][p]
  __shared__ __attribute__((aligned(16))) OT sR[RSZ];
  __shared__ float sS[QMAX];
  __shared__ float sDt[QMAX];
  __shared__ float sTmp[8];
  __shared__ float sRed[4][BQ][2];
  OT* const sDy = sR;
  OT* const sDyT = sR + IW * LDP;
  OT* const sGt = sR + IW * LDP + (BF ? PMAX * LDI : 0);
  OT* const sGam = sR;
  OT* const sGamT = sR + PMAX * LDN;
  OT* const sWt = sR;
  OT* const sCf = sR + BQ * LDI;

  const int nc = T / Q, nb = (Q + BQ - 1) / BQ;
  const int hpg = H / G, hps = hpg / nsplit;
  int idx = xcd_logical_block(blockIdx.x, gridDim.x);
  const int jb = idx % nb;
  idx /= nb;
  const int sp = idx % nsplit;
  idx /= nsplit;
  const int g = idx % G;
  idx /= G;
  const int c = idx % nc;
  const int bi = idx / nc;

  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), r = l & 15, q = l >> 4;
  const int64_t row0 = static_cast<int64_t>(bi) * T + static_cast<int64_t>(c) * Q;
  const int j0 = jb * BQ, vj = min(BQ, Q - j0);
  const int i_lo = j0;                          // rows i >= j0 feed this column block
  const int nsl = (Q - i_lo + IW - 1) / IW;     // slabs of i-rows
  const int Kn = round_up(N, Op<BF>::KS), Kp = round_up(P, Op<BF>::KS);
  const int64_t GN = static_cast<int64_t>(G) * N, HP = static_cast<int64_t>(H) * P;
  const int64_t PN = static_cast<int64_t>(P) * N;

  {
    RowTile<TI, BQ, NMAX> tb;
    tb.load(Bm + (row0 + j0) * GN + static_cast<int64_t>(g) * N, GN, vj, N);
    tb.store(sB, LDN);
  }
  f4 cb[NBMAX][4];
#pragma unroll
  for (int ib = 0; ib < NBMAX; ++ib) zero(cb[ib]);
  for (int sl = 0; sl < nsl; ++sl) {
    const int s0 = i_lo + sl * IW;
    RowTile<TI, IW, NMAX> tc;
    tc.load(Cm + (row0 + s0) * GN + static_cast<int64_t>(g) * N, GN, min(IW, Q - s0), N);
    __syncthreads();
    tc.store(sR, LDN);
    __syncthreads();
#pragma unroll
    for (int ib = 0; ib < NBMAX; ++ib) {
      const int il = ib * BQ - s0;
      if (ib >= jb && ib < nb && il >= 0 && il < IW)
        wave_gemm<BF, true, true, 4>(cb[ib], sR + (il + 16 * w) * LDN, LDN, 1, sB, LDN, 1, Kn);
    }
  }
  f4 ws[NBMAX][4];
#pragma unroll
  for (int ib = 0; ib < NBMAX; ++ib) zero(ws[ib]);
  f4 dbs[8];
  zero(dbs);

  RowTile<TI, BQ, PMAX> tX;          // x_jb
  // bf16 operands need dy and Gamma also transposed; f32 operands read the
  // transposed views with strided fetches, so rows suffice.
  typename std::conditional<BF, TransTile<TY, IW, PMAX>, RowTile<TY, IW, PMAX>>::type tDy;  // dy rows of a slab
  typename std::conditional<BF, TransTile<OT, PMAX, NMAX>, RowTile<OT, PMAX, NMAX>>::type tG;  // Gamma_{c+1}
  float dt_next = 0.f;
  auto load_head = [&](int hh) {
    const int h = g * hpg + sp * hps + hh;
    tX.load(x + (row0 + j0) * HP + static_cast<int64_t>(h) * P, HP, vj, P);
    tDy.load(dy + (row0 + i_lo) * HP + static_cast<int64_t>(h) * P, HP, min(IW, Q - i_lo), P);
    dt_next = (tid < Q) ? load_f(dt, (row0 + tid) * H + h) : 0.f;
  };
  load_head(0);

  for (int hh = 0; hh < hps; ++hh) {
    const int h = g * hpg + sp * hps + hh;
    const float A = -__expf(A_log[h]);
    const float Dh = D[h];
    const float dtv = dt_next;
    __syncthreads();  // previous head done with every tile
    const float s = block_inclusive_scan(dtv * A, sTmp);
    if (tid < Q) {
      sS[tid] = s;
      sDt[tid] = dtv;
    }
    tX.store(sX, LDP);
    // skip term D dy_j of this wave's output rows, loaded now, used at the end
    float dsk[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jq = j0 + 16 * w + 4 * q + i;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int p = 16 * t + r;
        dsk[i][t] = (jq < Q && p < P) ? load_f(dy, (row0 + jq) * HP + static_cast<int64_t>(h) * P + p) : 0.f;
      }
    }

    f4 dxa[4];
    zero(dxa);
    float csum[4] = {0.f, 0.f, 0.f, 0.f}, dsum[4] = {0.f, 0.f, 0.f, 0.f};
    bool sj_loaded = false;
    float sj[4], dtj4[4];
    for (int sl = 0; sl < nsl; ++sl) {
      const int s0 = i_lo + sl * IW;
      if (sl > 0) __syncthreads();
      tDy.store_rows(sDy, LDP);
      if constexpr (BF) tDy.store(sDyT, LDI);
      if (sl + 1 < nsl)
        tDy.load(dy + (row0 + s0 + IW) * HP + static_cast<int64_t>(h) * P, HP, min(IW, Q - s0 - IW), P);
      else
        tG.load(gamma + ((static_cast<int64_t>(bi) * nc + c) * H + h) * PN, N, P, N);
      __syncthreads();
#pragma unroll
      for (int ib = 0; ib < NBMAX; ++ib) {
        const int il = ib * BQ - s0;
        if (ib >= jb && ib < nb && il >= 0 && il < IW) {
          f4 yx[4];
          zero(yx);
          wave_gemm<BF, true, true, 4>(yx, sDy + (il + 16 * w) * LDP, LDP, 1, sX, LDP, 1, Kp);
          if (!sj_loaded) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
              const int jq = min(j0 + 16 * ct + r, Q - 1);
              sj[ct] = sS[jq];
              dtj4[ct] = sDt[jq];
            }
            sj_loaded = true;
          }
          const int ir0 = il + 16 * w + 4 * q;  // the lane's four rows inside the slab
          float si[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) si[i] = sS[min(s0 + ir0 + i, Q - 1)];
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            const int jl = 16 * ct + r, jq = j0 + jl;
            float g4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int iq = s0 + ir0 + i;
              const bool valid = iq < Q && jq <= iq;
              const float Lv = valid ? __expf(si[i] - sj[ct]) : 0.f;
              const float g1 = Lv * cb[ib][ct][i];
              const float e = g1 * yx[ct][i];
              csum[ct] += e;
              if (iq == jq) dsum[ct] += e;
              ws[ib][ct][i] += Lv * yx[ct][i] * dtj4[ct];
              g4[i] = g1;
            }
            OT* gp = sGt + jl * LDI + ir0;
            if constexpr (BF)
              *reinterpret_cast<uint2*>(gp) = make_uint2(pack_bf16(g4[0], g4[1]), pack_bf16(g4[2], g4[3]));
            else
              *reinterpret_cast<float4*>(gp) = make_float4(g4[0], g4[1], g4[2], g4[3]);
          }
        }
      }
      __syncthreads();
      const int kw = round_up(min(IW, Q - s0), Op<BF>::KS);
      if constexpr (BF)
        wave_gemm<BF, true, true, 4>(dxa, sGt + 16 * w * LDI, LDI, 1, sDyT, LDI, 1, kw);
      else
        wave_gemm<BF, true, false, 4>(dxa, sGt + 16 * w * LDI, LDI, 1, sDy, 1, LDP, kw);
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const float cs = sum_q(csum[ct]), ds = sum_q(dsum[ct]);
      if (q == 0) {
        sRed[w][16 * ct + r][0] = cs;
        sRed[w][16 * ct + r][1] = ds;
      }
    }

    // state terms with Gamma_{c+1}
    __syncthreads();
    tG.store_rows(sGam, LDN);
    if constexpr (BF) tG.store(sGamT, LDP);
    if (hh + 1 < hps) load_head(hh + 1);
    __syncthreads();
    if (tid < BQ && j0 + tid < Q) {
      const int64_t o = (static_cast<int64_t>(bi) * H + h) * T + static_cast<int64_t>(c) * Q + j0 + tid;
      colE[o] = sRed[0][tid][0] + sRed[1][tid][0] + sRed[2][tid][0] + sRed[3][tid][0];
      diagE[o] = sRed[0][tid][1] + sRed[1][tid][1] + sRed[2][tid][1] + sRed[3][tid][1];
    }
    f4 bg[4];
    zero(bg);
    wave_gemm<BF, true, true, 4>(bg, sB + 16 * w * LDN, LDN, 1, sGam, LDN, 1, Kn);
    f4 v[8];
    zero(v);
    if constexpr (BF)
      wave_gemm<BF, true, true, 8>(v, sX + 16 * w * LDP, LDP, 1, sGamT, LDP, 1, Kp);
    else
      wave_gemm<BF, true, false, 8>(v, sX + 16 * w * LDP, LDP, 1, sGam, 1, LDN, Kp);
    const float s_end = sS[Q - 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jl = 16 * w + 4 * q + i, jq = j0 + jl;
      const bool valid = jq < Q;
      const float wj = valid ? __expf(s_end - sS[jq]) : 0.f;
      const float dtj = valid ? sDt[jq] : 0.f;
      float part = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        part += v[t][i] * Op<BF>::back(sB[jl * LDN + 16 * t + r]);
        dbs[t][i] += dtj * wj * v[t][i];
      }
      part = sum16(part);
      if (valid && r == 0) Rp[(static_cast<int64_t>(bi) * H + h) * T + static_cast<int64_t>(c) * Q + jq] = wj * part;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int p = 16 * t + r;
        if (valid && p < P) {
          const int64_t o = (row0 + jq) * HP + static_cast<int64_t>(h) * P + p;
          dx[o] = dtj * (dxa[t][i] + wj * bg[t][i]) + Dh * dsk[i][t];
        }
      }
    }
  }

  // dB_j += sum_i W^T[j][i] C_i with W = sum over heads of L yx dt
  for (int sl = 0; sl < nsl; ++sl) {
    const int s0 = i_lo + sl * IW;
    __syncthreads();
#pragma unroll
    for (int ib = 0; ib < NBMAX; ++ib) {
      const int il = ib * BQ - s0;
      if (ib >= jb && ib < nb && il >= 0 && il < IW) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          OT* wp = sWt + (16 * ct + r) * LDI + il + 16 * w + 4 * q;
          if constexpr (BF)
            *reinterpret_cast<uint2*>(wp) = make_uint2(pack_bf16(ws[ib][ct][0], ws[ib][ct][1]),
                                                        pack_bf16(ws[ib][ct][2], ws[ib][ct][3]));
          else
            *reinterpret_cast<float4*>(wp) = make_float4(ws[ib][ct][0], ws[ib][ct][1], ws[ib][ct][2], ws[ib][ct][3]);
        }
      }
    }
    const int vi = min(IW, Q - s0);
    const TI* csrc = Cm + (row0 + s0) * GN + static_cast<int64_t>(g) * N;
    if constexpr (BF) {
      TransTile<TI, IW, NMAX> tc;
      tc.load(csrc, GN, vi, N);
      tc.store(sCf, LDI);
    } else {
      RowTile<TI, IW, NMAX> tc;
      tc.load(csrc, GN, vi, N);
      tc.store(sCf, LDN);
    }
    __syncthreads();
    const int kw = round_up(vi, Op<BF>::KS);
    if constexpr (BF)
      wave_gemm<BF, true, true, 8>(dbs, sWt + 16 * w * LDI, LDI, 1, sCf, LDI, 1, kw);
    else
      wave_gemm<BF, true, false, 8>(dbs, sWt + 16 * w * LDI, LDI, 1, sCf, 1, LDN, kw);
  }
  const int64_t batch = gridDim.x / (nb * nsplit * G * nc);
  float* dBo = dB_out + static_cast<int64_t>(sp) * batch * T * GN;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jq = j0 + 16 * w + 4 * q + i, n = 16 * t + r;
      if (jq < Q && n < N) dBo[(row0 + jq) * GN + static_cast<int64_t>(g) * N + n] = dbs[t][i];
    }
}

// --------------------------------------------------------------- row kernel

template <typename TI, typename TY, bool BF>
__global__ __launch_bounds__(NTHREADS) void chunk_bwd_row_kernel(
    const TI* __restrict__ x, const TI* __restrict__ Bm, const TI* __restrict__ Cm,
    const TI* __restrict__ dt, const TY* __restrict__ dy, const float* __restrict__ A_log,
    const float* __restrict__ hstates, float* __restrict__ dC_out, float* __restrict__ rowM,
    float* __restrict__ dsoff, float* __restrict__ dD_part, int T, int H, int P, int N, int G, int Q,
    int nsplit) {
  typedef typename Op<BF>::T OT;
  constexpr int PAD = BF ? 8 : 4;
  constexpr int JW = BwdSlab<BF>::W;
  constexpr int LDN = NMAX + PAD, LDP = PMAX + PAD, LDJ = JW + PAD;
  constexpr int R_PH1 = JW * LDN;                                        // B rows [j][n]
  constexpr int R_HEAD = (BF ? NMAX * LDP : PMAX * LDN) + JW * LDP;      // H^T [n][p] or H [p][n]; x rows [j][p]
  constexpr int R_FIN = BQ * LDJ + (BF ? NMAX * LDJ : JW * LDN);         // W [i][j]; B^T [n][j] or B [j][n]
  constexpr int RSZ = cmax(R_PH1, cmax(R_HEAD, R_FIN));
  __shared__ __attribute__((aligned(16))) OT sC[BQ * LDN];   // C_ib [i][n]
  __shared__ __attribute__((aligned(16))) OT sDy[BQ * LDP];  // dy_ib [i][p]
  __shared__ __attribute__((aligned(16))) OT sR[RSZ];
  __shared__ float sS[QMAX];
  __shared__ float sDt[QMAX];
  __shared__ float sTmp[8];
  OT* const sH = sR;
  OT* const sXr = sR + (BF ? NMAX * LDP : PMAX * LDN);
  OT* const sW = sR;
  OT* const sBf = sR + BQ * LDJ;

  const int nc = T / Q, nb = (Q + BQ - 1) / BQ;
  const int hpg = H / G, hps = hpg / nsplit;
  int idx = xcd_logical_block(blockIdx.x, gridDim.x);
  const int ib = nb - 1 - idx % nb;  // heavier row blocks first
  idx /= nb;
  const int sp = idx % nsplit;
  idx /= nsplit;
  const int g = idx % G;
  idx /= G;
  const int c = idx % nc;
  const int bi = idx / nc;

  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), r = l & 15, q = l >> 4;
  const int64_t row0 = static_cast<int64_t>(bi) * T + static_cast<int64_t>(c) * Q;
  const int i0 = ib * BQ, vi = min(BQ, Q - i0);
  const int jend = min(Q, i0 + BQ);
  const int nsl = (jend + JW - 1) / JW;
  const int Kn = round_up(N, Op<BF>::KS), Kp = round_up(P, Op<BF>::KS);
  const int64_t GN = static_cast<int64_t>(G) * N, HP = static_cast<int64_t>(H) * P;
  const int64_t PN = static_cast<int64_t>(P) * N;

  {
    RowTile<TI, BQ, NMAX> tc;
    tc.load(Cm + (row0 + i0) * GN + static_cast<int64_t>(g) * N, GN, vi, N);
    tc.store(sC, LDN);
  }
  f4 cb[NBMAX][4];
#pragma unroll
  for (int jb = 0; jb < NBMAX; ++jb) zero(cb[jb]);
  for (int sl = 0; sl < nsl; ++sl) {
    const int s0 = sl * JW;
    RowTile<TI, JW, NMAX> tb;
    tb.load(Bm + (row0 + s0) * GN + static_cast<int64_t>(g) * N, GN, min(JW, jend - s0), N);
    __syncthreads();
    tb.store(sR, LDN);
    __syncthreads();
#pragma unroll
    for (int jb = 0; jb < NBMAX; ++jb) {
      const int jl = jb * BQ - s0;
      if (jb <= ib && jl >= 0 && jl < JW)
        wave_gemm<BF, true, true, 4>(cb[jb], sC + 16 * w * LDN, LDN, 1, sR + jl * LDN, LDN, 1, Kn);
    }
  }
  f4 ws[NBMAX][4];
#pragma unroll
  for (int jb = 0; jb < NBMAX; ++jb) zero(ws[jb]);
  f4 dca[8];
  zero(dca);

  RowTile<TY, BQ, PMAX> tDy;        // dy_ib
  TransTile<float, PMAX, NMAX, 4> tH;  // H_c rows p, columns n
  RowTile<TI, JW, PMAX> tXs;        // x rows of one slab
  float dt_next = 0.f;
  auto load_head = [&](int hh) {
    const int h = g * hpg + sp * hps + hh;
    tDy.load(dy + (row0 + i0) * HP + static_cast<int64_t>(h) * P, HP, vi, P);
    tH.load(hstates + ((static_cast<int64_t>(bi) * nc + c) * H + h) * PN, N, P, N);
    tXs.load(x + row0 * HP + static_cast<int64_t>(h) * P, HP, min(JW, jend), P);
    dt_next = (tid < Q) ? load_f(dt, (row0 + tid) * H + h) : 0.f;
  };
  load_head(0);

  for (int hh = 0; hh < hps; ++hh) {
    const int h = g * hpg + sp * hps + hh;
    const float A = -__expf(A_log[h]);
    const float dtv = dt_next;
    __syncthreads();
    const float s = block_inclusive_scan(dtv * A, sTmp);
    if (tid < Q) {
      sS[tid] = s;
      sDt[tid] = dtv;
    }
    tDy.store(sDy, LDP);
    if constexpr (BF)
      tH.store(sH, LDP);
    else
      tH.store_rows(sH, LDN);
    __syncthreads();

    // U_i = dy_i H_c (rows i, d_state columns)
    f4 u[8];
    zero(u);
    if constexpr (BF)
      wave_gemm<BF, true, true, 8>(u, sDy + 16 * w * LDP, LDP, 1, sH, LDP, 1, Kp);
    else
      wave_gemm<BF, true, false, 8>(u, sDy + 16 * w * LDP, LDP, 1, sH, 1, LDN, Kp);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int il = 16 * w + 4 * q + i, iq = i0 + il;
      const float e = (iq < Q) ? __expf(sS[iq]) : 0.f;
      float part = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        part += u[t][i] * Op<BF>::back(sC[il * LDN + 16 * t + r]);
        dca[t][i] += e * u[t][i];
      }
      part = sum16(part);
      if (iq < Q && r == 0) dsoff[(static_cast<int64_t>(bi) * H + h) * T + static_cast<int64_t>(c) * Q + iq] = e * part;
    }

    float racc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int sl = 0; sl < nsl; ++sl) {
      const int s0 = sl * JW;
      __syncthreads();  // previous slab's reads of sXr done (and U's reads of sH)
      tXs.store(sXr, LDP);
      if (sl + 1 < nsl)
        tXs.load(x + (row0 + s0 + JW) * HP + static_cast<int64_t>(h) * P, HP, min(JW, jend - s0 - JW), P);
      else if (hh + 1 < hps)
        load_head(hh + 1);
      __syncthreads();
#pragma unroll
      for (int jb = 0; jb < NBMAX; ++jb) {
        const int jl = jb * BQ - s0;
        if (jb <= ib && jl >= 0 && jl < JW) {
          f4 yx[4];
          zero(yx);
          wave_gemm<BF, true, true, 4>(yx, sDy + 16 * w * LDP, LDP, 1, sXr + jl * LDP, LDP, 1, Kp);
          float si[4], sjv[4], dtjv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) si[i] = sS[min(i0 + 16 * w + 4 * q + i, Q - 1)];
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            const int jq = min(jb * BQ + 16 * ct + r, Q - 1);
            sjv[ct] = sS[jq];
            dtjv[ct] = sDt[jq];
          }
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int iq = i0 + 16 * w + 4 * q + i, jq = jb * BQ + 16 * ct + r;
              const bool valid = iq < Q && jq <= iq;
              const float ly = valid ? __expf(si[i] - sjv[ct]) * yx[ct][i] * dtjv[ct] : 0.f;
              ws[jb][ct][i] += ly;
              if (jq < iq) racc[i] += ly * cb[jb][ct][i];
            }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float rr = sum16(racc[i]);
      const int iq = i0 + 16 * w + 4 * q + i;
      if (iq < Q && r == 0) rowM[(static_cast<int64_t>(bi) * H + h) * T + static_cast<int64_t>(c) * Q + iq] = rr;
    }
    // dD partial over this block's rows
    float dd = 0.f;
    for (int e = tid; e < vi * P; e += NTHREADS) {
      const int il = e / P, p = e % P;
      const int64_t o = (row0 + i0 + il) * HP + static_cast<int64_t>(h) * P + p;
      dd += load_f(dy, o) * load_f(x, o);
    }
    dd = wave_sum(dd);
    if (l == 0) sTmp[4 + w] = dd;
    __syncthreads();
    if (tid == 0) dD_part[((static_cast<int64_t>(bi) * nc + c) * nb + ib) * H + h] = sTmp[4] + sTmp[5] + sTmp[6] + sTmp[7];
  }

  // dC_i += sum_j W[i][j] B_j with W = sum over heads of L yx dt
  for (int sl = 0; sl < nsl; ++sl) {
    const int s0 = sl * JW;
    __syncthreads();
#pragma unroll
    for (int jb = 0; jb < NBMAX; ++jb) {
      const int jl = jb * BQ - s0;
      if (jb <= ib && jl >= 0 && jl < JW) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sW[(16 * w + 4 * q + i) * LDJ + jl + 16 * ct + r] = Op<BF>::cvt(ws[jb][ct][i]);
      }
    }
    const int vj = min(JW, jend - s0);
    const TI* bsrc = Bm + (row0 + s0) * GN + static_cast<int64_t>(g) * N;
    if constexpr (BF) {
      TransTile<TI, JW, NMAX> tb;
      tb.load(bsrc, GN, vj, N);
      tb.store(sBf, LDJ);
    } else {
      RowTile<TI, JW, NMAX> tb;
      tb.load(bsrc, GN, vj, N);
      tb.store(sBf, LDN);
    }
    __syncthreads();
    const int kw = round_up(vj, Op<BF>::KS);
    if constexpr (BF)
      wave_gemm<BF, true, true, 8>(dca, sW + 16 * w * LDJ, LDJ, 1, sBf, LDJ, 1, kw);
    else
      wave_gemm<BF, true, false, 8>(dca, sW + 16 * w * LDJ, LDJ, 1, sBf, 1, LDN, kw);
  }
  const int64_t batch = gridDim.x / (nb * nsplit * G * nc);
  float* dCo = dC_out + static_cast<int64_t>(sp) * batch * T * GN;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int iq = i0 + 16 * w + 4 * q + i, n = 16 * t + r;
      if (iq < Q && n < N) dCo[(row0 + iq) * GN + static_cast<int64_t>(g) * N + n] = dca[t][i];
    }
}

// ------------------------------------------------------------- dt finalize

template <typename TI>
__global__ __launch_bounds__(NTHREADS) void bwd_dt_kernel(const TI* __restrict__ dt, const float* __restrict__ A_log,
                                                          float* __restrict__ ddt, BwdScratch s, int T, int H, int Q,
                                                          int npb) {
  __shared__ float sTmp[8];
  __shared__ float sLast;
  const int c = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  const int nc = gridDim.x;
  const int k = threadIdx.x;
  const bool valid = k < Q;
  const int64_t t0 = static_cast<int64_t>(c) * Q;
  const float A = -__expf(A_log[h]);
  const float dtv = valid ? load_f(dt, (static_cast<int64_t>(bi) * T + t0 + k) * H + h) : 0.f;
  const float sv = block_inclusive_scan(dtv * A, sTmp);
  if (k == Q - 1) sLast = sv;
  const int64_t o = (static_cast<int64_t>(bi) * H + h) * T + t0 + k;
  float colE = 0.f, Rp = 0.f, ds = 0.f;
  if (valid) {
    colE = s.colE[o];
    Rp = s.Rp[o];
    ds = s.rowM[o] - dtv * (colE - s.diagE[o]) + s.dsoff[o] - dtv * Rp;
  }
  const float totR = block_sum(dtv * Rp, sTmp);  // syncs make sLast visible
  if (k == Q - 1) {
    float gh = 0.f;
    const float* ghp = s.gh_part + ((static_cast<int64_t>(bi) * nc + c) * H + h) * npb;
    for (int pb = 0; pb < npb; ++pb) gh += ghp[pb];
    ds += totR + __expf(sLast) * gh;
  }
  const float incl = block_inclusive_scan(ds, sTmp);
  __syncthreads();
  if (k == Q - 1) sLast = incl;
  __syncthreads();
  const float da = sLast - incl + ds;  // sum_{k' >= k} ds_k'
  if (valid) ddt[(static_cast<int64_t>(bi) * T + t0 + k) * H + h] = colE + Rp + A * da;
  const float dA = block_sum(dtv * da, sTmp);
  if (k == 0) s.dA_part[(static_cast<int64_t>(bi) * nc + c) * H + h] = dA;
}

// ----------------------------------------------------------- final sums

__global__ __launch_bounds__(NTHREADS) void bwd_param_reduce_kernel(const float* __restrict__ A_log,
                                                                    float* __restrict__ dA_log,
                                                                    float* __restrict__ dD, BwdScratch s, int nbc,
                                                                    int nb, int H) {
  __shared__ float sTmp[8];
  const int h = blockIdx.x;
  float a = 0.f, dd = 0.f;
  for (int u = threadIdx.x; u < nbc; u += NTHREADS) {
    a += s.dA_part[static_cast<int64_t>(u) * H + h];
    for (int ib = 0; ib < nb; ++ib) dd += s.dD_part[(static_cast<int64_t>(u) * nb + ib) * H + h];
  }
  a = block_sum(a, sTmp);
  dd = block_sum(dd, sTmp);
  if (threadIdx.x == 0) {
    dA_log[h] = -__expf(A_log[h]) * a;
    dD[h] = dd;
  }
}

__global__ void split_sum_kernel(const float* __restrict__ part, float* __restrict__ out, int64_t n, int nsplit) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float acc = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) acc += part[static_cast<int64_t>(sp) * n + i];
  out[i] = acc;
}

__global__ void fill_kernel(float* __restrict__ p, int64_t n, float v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void copy_kernel(float* __restrict__ dst, const float* __restrict__ src, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

// ---------------------------------------------------------------- launchers

static int64_t nblocks_chunk(const Dims& d, int nsplit) {
  return static_cast<int64_t>(d.b) * d.nc() * d.G * nsplit * d.nb();
}

template <typename TI, typename TY, bool BF>
static void col_launch(const Dims& d, int nsplit, const void* x, const void* B, const void* C, const void* dt,
                       const void* dy, const float* A_log, const float* D, const void* gamma, float* dx,
                       float* dB_out, const BwdScratch& s, hipStream_t st) {
  hipLaunchKernelGGL((chunk_bwd_col_kernel<TI, TY, BF>), dim3(nblocks_chunk(d, nsplit)), dim3(NTHREADS), 0, st,
                     static_cast<const TI*>(x), static_cast<const TI*>(B), static_cast<const TI*>(C),
                     static_cast<const TI*>(dt), static_cast<const TY*>(dy), A_log, D,
                     static_cast<const typename Op<BF>::T*>(gamma), dx, dB_out, s.colE,
                     s.diagE, s.Rp, d.T, d.H, d.P, d.N, d.G, d.Q, nsplit);
}

hipError_t launch_chunk_bwd_col(const Dims& d, DType act, DType dyt, int nsplit, const void* x,
                                const void* B, const void* C, const void* dt, const void* dy,
                                const float* A_log, const float* D, const void* gamma, float* dx,
                                float* dB_out, const BwdScratch& s, hipStream_t st) {
  if (act == BF16) {
    if (dyt == BF16)
      col_launch<uint16_t, uint16_t, true>(d, nsplit, x, B, C, dt, dy, A_log, D, gamma, dx, dB_out, s, st);
    else
      col_launch<uint16_t, float, true>(d, nsplit, x, B, C, dt, dy, A_log, D, gamma, dx, dB_out, s, st);
  } else {
    if (dyt == BF16)
      col_launch<float, uint16_t, false>(d, nsplit, x, B, C, dt, dy, A_log, D, gamma, dx, dB_out, s, st);
    else
      col_launch<float, float, false>(d, nsplit, x, B, C, dt, dy, A_log, D, gamma, dx, dB_out, s, st);
  }
  return hipGetLastError();
}

template <typename TI, typename TY, bool BF>
static void row_launch(const Dims& d, int nsplit, const void* x, const void* B, const void* C, const void* dt,
                       const void* dy, const float* A_log, const float* states, float* dC_out, const BwdScratch& s,
                       hipStream_t st) {
  hipLaunchKernelGGL((chunk_bwd_row_kernel<TI, TY, BF>), dim3(nblocks_chunk(d, nsplit)), dim3(NTHREADS), 0, st,
                     static_cast<const TI*>(x), static_cast<const TI*>(B), static_cast<const TI*>(C),
                     static_cast<const TI*>(dt), static_cast<const TY*>(dy), A_log, states, dC_out, s.rowM, s.dsoff,
                     s.dD_part, d.T, d.H, d.P, d.N, d.G, d.Q, nsplit);
}

hipError_t launch_chunk_bwd_row(const Dims& d, DType act, DType dyt, int nsplit, const void* x,
                                const void* B, const void* C, const void* dt, const void* dy,
                                const float* A_log, const float* states, float* dC_out,
                                const BwdScratch& s, hipStream_t st) {
  if (act == BF16) {
    if (dyt == BF16)
      row_launch<uint16_t, uint16_t, true>(d, nsplit, x, B, C, dt, dy, A_log, states, dC_out, s, st);
    else
      row_launch<uint16_t, float, true>(d, nsplit, x, B, C, dt, dy, A_log, states, dC_out, s, st);
  } else {
    if (dyt == BF16)
      row_launch<float, uint16_t, false>(d, nsplit, x, B, C, dt, dy, A_log, states, dC_out, s, st);
    else
      row_launch<float, float, false>(d, nsplit, x, B, C, dt, dy, A_log, states, dC_out, s, st);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dt(const Dims& d, DType act, const void* dt, const float* A_log, float* ddt,
                         const BwdScratch& s, hipStream_t st) {
  dim3 grid(d.nc(), d.H, d.b);
  if (act == BF16)
    hipLaunchKernelGGL((bwd_dt_kernel<uint16_t>), grid, dim3(NTHREADS), 0, st, static_cast<const uint16_t*>(dt),
                       A_log, ddt, s, d.T, d.H, d.Q, state_npb(d));
  else
    hipLaunchKernelGGL((bwd_dt_kernel<float>), grid, dim3(NTHREADS), 0, st, static_cast<const float*>(dt), A_log,
                       ddt, s, d.T, d.H, d.Q, state_npb(d));
  return hipGetLastError();
}

hipError_t launch_bwd_reduce(const Dims& d, int nsplit, const float* A_log, float* dA_log,
                             float* dD, float* dB, float* dC, const BwdScratch& s, hipStream_t st) {
  hipLaunchKernelGGL(bwd_param_reduce_kernel, dim3(d.H), dim3(NTHREADS), 0, st, A_log, dA_log, dD, s,
                     d.b * d.nc(), d.nb(), d.H);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  const int64_t n = static_cast<int64_t>(d.b) * d.T * d.G * d.N;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(split_sum_kernel, dim3(blocks), dim3(256), 0, st, s.dB_part, dB, n, nsplit);
  hipLaunchKernelGGL(split_sum_kernel, dim3(blocks), dim3(256), 0, st, s.dC_part, dC, n, nsplit);
  return hipGetLastError();
}

hipError_t launch_fill(float* p, int64_t n, float value, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n, value);
  return hipGetLastError();
}

hipError_t launch_copy(float* dst, const float* src, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_kernel, dim3((n + 255) / 256), dim3(256), 0, st, dst, src, n);
  return hipGetLastError();
}

}  // namespace ssd
