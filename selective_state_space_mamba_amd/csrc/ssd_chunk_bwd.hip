// Intra-chunk backward of the SSD and the dt / A / D reductions.
//
// Gradients of L = sum(dy * y) for one chunk follow from the reverse-time loop
// of the reference page (burn_dragon_kernel src/sequence/mamba2/backward.rs,
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

#include "ssd_async.hpp"
#include "ssd_common.hpp"
#include "ssd_launch.hpp"

namespace ssd {

// Sum over the workgroup; result valid in every thread.  `tmp`: 4 floats.
// Ends with a barrier, so the next user of `tmp` (a scan writes it before its
// first barrier) cannot overwrite the partial sums while a wave still reads them.
__device__ __forceinline__ float block_sum(float v, float* tmp) {
  v = wave_sum(v);
  __syncthreads();
  if (lane_id() == 0) tmp[wave_id()] = v;
  __syncthreads();
  const float total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  __syncthreads();
  return total;
}

// Chunk rows (or columns) staged per slab: 128 at a time for bf16 operands, 64
// for f32.
template <bool BF> struct BwdSlab { static constexpr int W = BF ? 2 * BQ : BQ; };

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// ------------------------------------------------------------ column kernel
//
// 8 waves; wave w = (rw, cw) with rw = w % 4, cw = w / 4 owns rows 16*rw..+15
// and columns 32*cw..+31 of every 64 x 64 tile it computes (two 16-wide MFMA
// tiles), so two waves share each SIMD.

constexpr int NT8 = 512;

// PAIRED: a workgroup takes column blocks k and then nb - 1 - k (its own
// instantiation: the pass loop costs registers that the one-block form keeps)
template <typename TI, typename TY, bool BF, bool PAIRED>
__global__ __launch_bounds__(NT8) void chunk_bwd_col_kernel(
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
  __shared__ float sTmp[16];
  __shared__ float sRed[4][BQ][2];
  __shared__ float sRp[2][BQ];
  // bf16 mode keeps the sum over heads of L yx dt for every tile in LDS (f32,
  // each lane owning the 8 values of its two 16x16 fragments, so no two lanes
  // touch a slot) to stay within two waves' registers; f32 mode keeps it in
  // registers (its tiles leave no LDS for it).
  __shared__ __attribute__((aligned(16))) float sWs[BF ? NBMAX * NT8 * 8 : 4];
  f4 wsr[NBMAX][2];
  OT* const sDy = sR;
  OT* const sDyT = sR + IW * LDP;
  OT* const sGt = sR + IW * LDP + (BF ? PMAX * LDI : 0);
  OT* const sGam = sR;
  OT* const sGamT = sR + PMAX * LDN;
  OT* const sWt = sR;
  OT* const sCf = sR + BQ * LDI;

  const int nc = T / Q, nb = (Q + BQ - 1) / BQ;
  const int hpg = H / G, hps = hpg / nsplit;
  // paired: column blocks k and then nb - 1 - k, so that every workgroup has
  // the same number of (row block, column block) tiles; else one block
  const int nunit = PAIRED ? (nb + 1) >> 1 : nb;
  int idx = xcd_logical_block(blockIdx.x, gridDim.x);
  const int unit = idx % nunit;
  idx /= nunit;
  const int sp = idx % nsplit;
  idx /= nsplit;
  const int g = idx % G;
  idx /= G;
  const int c = idx % nc;
  const int bi = idx / nc;

  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), r = l & 15, q = l >> 4;
  const int rw = w & 3, cw = w >> 2;
  const int64_t row0 = static_cast<int64_t>(bi) * T + static_cast<int64_t>(c) * Q;
#pragma unroll 1
  for (int pass = 0; pass < (PAIRED ? 2 : 1); ++pass) {
  const int jb = pass ? nb - 1 - unit : unit;
  if (pass && jb == unit) break;
  if (pass) __syncthreads();  // the first block is done with every tile
  // paired: the lane indices taken afresh in each pass, so that offsets
  // derived from them are not hoisted out of the pass loop and held across it
  const int lp = PAIRED ? opaque_index(lane_id()) : lane_id();
  const int l = lp, r = lp & 15, q = lp >> 4;
  (void)l;
  const int j0 = jb * BQ, vj = min(BQ, Q - j0);
  const int i_lo = j0;                          // rows i >= j0 feed this column block
  const int nsl = (Q - i_lo + IW - 1) / IW;     // slabs of i-rows
  const int Kn = round_up(N, Op<BF>::KS), Kp = round_up(P, Op<BF>::KS);
  const int64_t GN = static_cast<int64_t>(G) * N, HP = static_cast<int64_t>(H) * P;
  const int64_t PN = static_cast<int64_t>(P) * N;

  {
    RowTile<TI, BQ, NMAX, NT8> tb;
    tb.load(Bm + (row0 + j0) * GN + static_cast<int64_t>(g) * N, GN, vj, N);
    tb.store(sB, LDN);
  }
  // C.B^T tiles (ib, jb): rows i (this wave's 16), columns j (this wave's 32)
  f4 cb[NBMAX][2];
#pragma unroll
  for (int ib = 0; ib < NBMAX; ++ib) zero(cb[ib]);
  for (int sl = 0; sl < nsl; ++sl) {
    const int s0 = i_lo + sl * IW;
    RowTile<TI, IW, NMAX, NT8> tc;
    tc.load(Cm + (row0 + s0) * GN + static_cast<int64_t>(g) * N, GN, min(IW, Q - s0), N);
    __syncthreads();
    tc.store(sR, LDN);
    __syncthreads();
#pragma unroll
    for (int ib = 0; ib < NBMAX; ++ib) {
      const int il = ib * BQ - s0;
      if (ib >= jb && ib < nb && il >= 0 && il < IW)
        wave_gemm<BF, true, true, 2>(cb[ib], sR + (il + 16 * rw) * LDN, LDN, 1, sB + 32 * cw * LDN, LDN, 1, Kn);
    }
  }
#pragma unroll
  for (int ib = 0; ib < NBMAX; ++ib) {
    zero(wsr[ib]);
    if constexpr (BF) {
      float4* wsp = reinterpret_cast<float4*>(sWs + (ib * NT8 + tid) * 8);
      wsp[0] = make_float4(0.f, 0.f, 0.f, 0.f);
      wsp[1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  f4 dbs[4];        // dB rows j (16 rw), columns n 64*cw..+63
  zero(dbs);

  // bf16 operands need dy and Gamma also transposed; f32 operands read the
  // transposed views with strided fetches, so rows suffice.
  RowTile<TI, BQ, PMAX, NT8> tX;
  typename std::conditional<BF, TransTile<TY, IW, PMAX, 4, NT8>, RowTile<TY, IW, PMAX, NT8>>::type tDy;
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
    f4 dxa[2];
    zero(dxa);
    float csum[2] = {0.f, 0.f}, dsum[2] = {0.f, 0.f};
    float sj[2], dtj2[2];
    for (int sl = 0; sl < nsl; ++sl) {
      const int s0 = i_lo + sl * IW;
      if (sl > 0) __syncthreads();
      tDy.store_rows(sDy, LDP);
      if constexpr (BF) tDy.store(sDyT, LDI);
      if (sl + 1 < nsl)
        tDy.load(dy + (row0 + s0 + IW) * HP + static_cast<int64_t>(h) * P, HP, min(IW, Q - s0 - IW), P);
      __syncthreads();
      if (sl == 0) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int jq = min(j0 + 32 * cw + 16 * t + r, Q - 1);
          sj[t] = sS[jq];
          dtj2[t] = sDt[jq];
        }
      }
#pragma unroll
      for (int ib = 0; ib < NBMAX; ++ib) {
        const int il = ib * BQ - s0;
        if (ib >= jb && ib < nb && il >= 0 && il < IW) {
          f4 yx[2];
          zero(yx);
          wave_gemm<BF, true, true, 2>(yx, sDy + (il + 16 * rw) * LDP, LDP, 1, sX + 32 * cw * LDP, LDP, 1, Kp);
          float4* wsp = reinterpret_cast<float4*>(sWs + (ib * NT8 + tid) * 8);
          f4 ws[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if constexpr (BF) {
              const float4 v4 = wsp[t];
              ws[t] = f4{v4.x, v4.y, v4.z, v4.w};
            } else {
              ws[t] = wsr[ib][t];
            }
          }
          // the lane index taken here: masks and offsets built from it once
          // for the whole head loop would be spilled (one lane mask per
          // (block, tile, element))
          const int lo = opaque_index(lane_id()), ro = lo & 15, qo = lo >> 4;
          const int ir0 = il + 16 * rw + 4 * qo;  // the lane's four rows inside the slab
          float si[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) si[e] = sS[min(s0 + ir0 + e, Q - 1)];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int jl = 32 * cw + 16 * t + ro, jq = j0 + jl;
            float g4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int iq = s0 + ir0 + e;
              const bool valid = iq < Q && jq <= iq;
              const float Lv = valid ? __expf(si[e] - sj[t]) : 0.f;
              const float g1 = Lv * cb[ib][t][e];
              const float E = g1 * yx[t][e];
              csum[t] += E;
              if (iq == jq) dsum[t] += E;
              ws[t][e] += Lv * yx[t][e] * dtj2[t];
              g4[e] = g1;
            }
            OT* gp = sGt + jl * LDI + ir0;
            if constexpr (BF)
              *reinterpret_cast<uint2*>(gp) = make_uint2(pack_bf16(g4[0], g4[1]), pack_bf16(g4[2], g4[3]));
            else
              *reinterpret_cast<float4*>(gp) = make_float4(g4[0], g4[1], g4[2], g4[3]);
          }
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if constexpr (BF)
              wsp[t] = make_float4(ws[t][0], ws[t][1], ws[t][2], ws[t][3]);
            else
              wsr[ib][t] = ws[t];
          }
        }
      }
      __syncthreads();
      const int kw = round_up(min(IW, Q - s0), Op<BF>::KS);
      if constexpr (BF)
        wave_gemm<BF, true, true, 2>(dxa, sGt + 16 * rw * LDI, LDI, 1, sDyT + 32 * cw * LDI, LDI, 1, kw);
      else
        wave_gemm<BF, true, false, 2>(dxa, sGt + 16 * rw * LDI, LDI, 1, sDy + 32 * cw, 1, LDP, kw);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float cs = sum_q(csum[t]), ds = sum_q(dsum[t]);
      if (q == 0) {
        sRed[rw][32 * cw + 16 * t + r][0] = cs;
        sRed[rw][32 * cw + 16 * t + r][1] = ds;
      }
    }

    // state terms with Gamma_{c+1}
    {
      typename std::conditional<BF, TransTile<OT, PMAX, NMAX, 4, NT8>, RowTile<OT, PMAX, NMAX, NT8>>::type tG;
      tG.load(gamma + ((static_cast<int64_t>(bi) * nc + c) * H + h) * PN, N, P, N);
      __syncthreads();
      tG.store_rows(sGam, LDN);
      if constexpr (BF) tG.store(sGamT, LDP);
    }
    if (hh + 1 < hps) load_head(hh + 1);
    __syncthreads();
    // the lane index taken per head (see the step loop): the row and column
    // masks of the skip loads, the state terms and the dx stores are built
    // here, not hoisted out of the head loop
    const int lh = opaque_index(lane_id()), rh = lh & 15, qh = lh >> 4;
    // skip term D dy_j (loaded here, while the MFMAs below run) for this wave's output rows j, columns p
    float dsk[4][2];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int jq = j0 + 16 * rw + 4 * qh + e;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int p = 32 * cw + 16 * t + rh;
        dsk[e][t] = (jq < Q && p < P) ? load_f(dy, (row0 + jq) * HP + static_cast<int64_t>(h) * P + p) : 0.f;
      }
    }

    if (tid < BQ && j0 + tid < Q) {
      const int64_t o = (static_cast<int64_t>(bi) * H + h) * T + static_cast<int64_t>(c) * Q + j0 + tid;
      colE[o] = sRed[0][tid][0] + sRed[1][tid][0] + sRed[2][tid][0] + sRed[3][tid][0];
      diagE[o] = sRed[0][tid][1] + sRed[1][tid][1] + sRed[2][tid][1] + sRed[3][tid][1];
    }
    // bg = B Gamma^T (rows j, columns p), v = x Gamma (rows j, columns n)
    f4 bg[2];
    zero(bg);
    wave_gemm<BF, true, true, 2>(bg, sB + 16 * rw * LDN, LDN, 1, sGam + 32 * cw * LDN, LDN, 1, Kn);
    f4 v[4];
    zero(v);
    if constexpr (BF)
      wave_gemm<BF, true, true, 4>(v, sX + 16 * rw * LDP, LDP, 1, sGamT + 64 * cw * LDP, LDP, 1, Kp);
    else
      wave_gemm<BF, true, false, 4>(v, sX + 16 * rw * LDP, LDP, 1, sGam + 64 * cw, 1, LDN, Kp);
    const float s_end = sS[Q - 1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int jl = 16 * rw + 4 * qh + e, jq = j0 + jl;
      const bool valid = jq < Q;
      const float wj = valid ? __expf(s_end - sS[jq]) : 0.f;
      const float dtj = valid ? sDt[jq] : 0.f;
      // R'_j / w_j = x_j . (B_j Gamma^T): partial over this wave's columns p
      float part = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) part += bg[t][e] * Op<BF>::back(sX[jl * LDP + 32 * cw + 16 * t + rh]);
      part = sum16(part);
      if (rh == 0) sRp[cw][jl] = part;
#pragma unroll
      for (int t = 0; t < 4; ++t) dbs[t][e] += dtj * wj * v[t][e];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int p = 32 * cw + 16 * t + rh;
        if (valid && p < P) {
          const int64_t o = (row0 + jq) * HP + static_cast<int64_t>(h) * P + p;
          dx[o] = dtj * (dxa[t][e] + wj * bg[t][e]) + Dh * dsk[e][t];
        }
      }
    }
    __syncthreads();
    if (tid < BQ && j0 + tid < Q)
      Rp[(static_cast<int64_t>(bi) * H + h) * T + static_cast<int64_t>(c) * Q + j0 + tid] =
          __expf(s_end - sS[j0 + tid]) * (sRp[0][tid] + sRp[1][tid]);
  }

  // dB_j += sum_i W^T[j][i] C_i with W = sum over heads of L yx dt
  for (int sl = 0; sl < nsl; ++sl) {
    const int s0 = i_lo + sl * IW;
    __syncthreads();
#pragma unroll
    for (int ib = 0; ib < NBMAX; ++ib) {
      const int il = ib * BQ - s0;
      if (ib >= jb && ib < nb && il >= 0 && il < IW) {
        const float4* wsp = reinterpret_cast<const float4*>(sWs + (ib * NT8 + tid) * 8);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float4 v4;
          if constexpr (BF)
            v4 = wsp[t];
          else
            v4 = make_float4(wsr[ib][t][0], wsr[ib][t][1], wsr[ib][t][2], wsr[ib][t][3]);
          OT* wp = sWt + (32 * cw + 16 * t + r) * LDI + il + 16 * rw + 4 * q;
          if constexpr (BF)
            *reinterpret_cast<uint2*>(wp) = make_uint2(pack_bf16(v4.x, v4.y), pack_bf16(v4.z, v4.w));
          else
            *reinterpret_cast<float4*>(wp) = v4;
        }
      }
    }
    const int vi = min(IW, Q - s0);
    const TI* csrc = Cm + (row0 + s0) * GN + static_cast<int64_t>(g) * N;
    if constexpr (BF) {
      TransTile<TI, IW, NMAX, 4, NT8> tc;
      tc.load(csrc, GN, vi, N);
      tc.store(sCf, LDI);
    } else {
      RowTile<TI, IW, NMAX, NT8> tc;
      tc.load(csrc, GN, vi, N);
      tc.store(sCf, LDN);
    }
    __syncthreads();
    const int kw = round_up(vi, Op<BF>::KS);
    if constexpr (BF)
      wave_gemm<BF, true, true, 4>(dbs, sWt + 16 * rw * LDI, LDI, 1, sCf + 64 * cw * LDI, LDI, 1, kw);
    else
      wave_gemm<BF, true, false, 4>(dbs, sWt + 16 * rw * LDI, LDI, 1, sCf + 64 * cw, 1, LDN, kw);
  }
  const int64_t batch = gridDim.x / (nunit * nsplit * G * nc);
  float* dBo = dB_out + static_cast<int64_t>(sp) * batch * T * GN;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int jq = j0 + 16 * rw + 4 * q + e, n = 64 * cw + 16 * t + r;
      if (jq < Q && n < N) dBo[(row0 + jq) * GN + static_cast<int64_t>(g) * N + n] = dbs[t][e];
    }
  }  // pass
}

// --------------------------------------------------------------- row kernel
//
// 8 waves.  The causal tiles are computed transposed (rows j, columns i):
// wave (rw, cw) owns rows j 16*rw..+15 and columns i 32*cw..+31 of each tile,
// so the head-summed W[i][j] is written to LDS with packed 8-byte stores.  The
// incoming-state term U = dy H_c (rows i, d_state columns) uses rows i 16*rw,
// columns n 64*cw..+63, as does dC.

// PAIRED: row blocks nb - 1 - k and then k (see the column kernel)
template <typename TI, typename TY, bool BF, bool PAIRED>
__global__ __launch_bounds__(NT8) void chunk_bwd_row_kernel(
    const TI* __restrict__ x, const TI* __restrict__ Bm, const TI* __restrict__ Cm,
    const TI* __restrict__ dt, const TY* __restrict__ dy, const float* __restrict__ A_log,
    const float* __restrict__ hstates, float* __restrict__ dC_out, float* __restrict__ rowM,
    float* __restrict__ dsoff, float* __restrict__ dD_part, unsigned* __restrict__ done, int T, int H, int P,
    int N, int G, int Q, int nsplit) {
  typedef typename Op<BF>::T OT;
  // the dt kernel that follows counts its finished workgroups from 0
  if (blockIdx.x == 0 && threadIdx.x == 0) __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

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
  __shared__ float sTmp[16];
  __shared__ float sRow[4][BQ];  // row sums of M by row group of j
  __shared__ float sDso[2][BQ];  // U_i . C_i by column half of n
  // bf16 mode keeps the head sum of L yx dt in LDS (each lane owns its slots);
  // f32 mode in registers.
  __shared__ __attribute__((aligned(16))) float sWs[BF ? NBMAX * NT8 * 8 : 4];
  OT* const sH = sR;
  OT* const sXr = sR + (BF ? NMAX * LDP : PMAX * LDN);
  OT* const sW = sR;
  OT* const sBf = sR + BQ * LDJ;

  const int nc = T / Q, nb = (Q + BQ - 1) / BQ;
  const int hpg = H / G, hps = hpg / nsplit;
  // paired: row blocks nb - 1 - k and then k (equal work per workgroup);
  // else one block, the heavier ones first
  const int nunit = PAIRED ? (nb + 1) >> 1 : nb;
  int idx = xcd_logical_block(blockIdx.x, gridDim.x);
  const int unit = idx % nunit;
  idx /= nunit;
  const int sp = idx % nsplit;
  idx /= nsplit;
  const int g = idx % G;
  idx /= G;
  const int c = idx % nc;
  const int bi = idx / nc;

  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), r = l & 15, q = l >> 4;
  const int rw = w & 3, cw = w >> 2;
  const int64_t row0 = static_cast<int64_t>(bi) * T + static_cast<int64_t>(c) * Q;
#pragma unroll 1
  for (int pass = 0; pass < (PAIRED ? 2 : 1); ++pass) {
  const int ib = pass ? unit : nb - 1 - unit;
  if (pass && ib == nb - 1 - unit) break;
  if (pass) __syncthreads();  // the first block is done with every tile
  // paired: the lane indices taken afresh in each pass (see the column kernel)
  const int lp = PAIRED ? opaque_index(lane_id()) : lane_id();
  const int l = lp, r = lp & 15, q = lp >> 4;
  (void)l;
  const int i0 = ib * BQ, vi = min(BQ, Q - i0);
  const int jend = min(Q, i0 + BQ);
  const int nsl = (jend + JW - 1) / JW;
  const int Kn = round_up(N, Op<BF>::KS), Kp = round_up(P, Op<BF>::KS);
  const int64_t GN = static_cast<int64_t>(G) * N, HP = static_cast<int64_t>(H) * P;
  const int64_t PN = static_cast<int64_t>(P) * N;

  {
    RowTile<TI, BQ, NMAX, NT8> tc;
    tc.load(Cm + (row0 + i0) * GN + static_cast<int64_t>(g) * N, GN, vi, N);
    tc.store(sC, LDN);
  }
  // (C.B^T)^T tiles (jb, ib): rows j (this wave's 16), columns i (this wave's 32)
  f4 cb[NBMAX][2];
#pragma unroll
  for (int jb = 0; jb < NBMAX; ++jb) zero(cb[jb]);
  for (int sl = 0; sl < nsl; ++sl) {
    const int s0 = sl * JW;
    RowTile<TI, JW, NMAX, NT8> tb;
    tb.load(Bm + (row0 + s0) * GN + static_cast<int64_t>(g) * N, GN, min(JW, jend - s0), N);
    __syncthreads();
    tb.store(sR, LDN);
    __syncthreads();
#pragma unroll
    for (int jb = 0; jb < NBMAX; ++jb) {
      const int jl = jb * BQ - s0;
      if (jb <= ib && jl >= 0 && jl < JW)
        wave_gemm<BF, true, true, 2>(cb[jb], sR + (jl + 16 * rw) * LDN, LDN, 1, sC + 32 * cw * LDN, LDN, 1, Kn);
    }
  }
  f4 wsr[NBMAX][2];  // sum over heads of L yx dt, transposed like cb (f32 mode)
#pragma unroll
  for (int jb = 0; jb < NBMAX; ++jb) {
    zero(wsr[jb]);
    if constexpr (BF) {
      float4* wsp = reinterpret_cast<float4*>(sWs + (jb * NT8 + tid) * 8);
      wsp[0] = make_float4(0.f, 0.f, 0.f, 0.f);
      wsp[1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  f4 dca[4];        // dC rows i (16 rw), columns n 64*cw..+63
  zero(dca);

  RowTile<TY, BQ, PMAX, NT8> tDy;  // dy_ib
  RowTile<TI, JW, PMAX, NT8> tXs;  // x rows of one slab
  float dt_next = 0.f;
  auto load_head = [&](int hh) {
    const int h = g * hpg + sp * hps + hh;
    tDy.load(dy + (row0 + i0) * HP + static_cast<int64_t>(h) * P, HP, vi, P);
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
    {
      typename std::conditional<BF, TransTile<float, PMAX, NMAX, 4, NT8>, RowTile<float, PMAX, NMAX, NT8>>::type tH;
      tH.load(hstates + ((static_cast<int64_t>(bi) * nc + c) * H + h) * PN, N, P, N);
      if constexpr (BF)
        tH.store(sH, LDP);
      else
        tH.store_rows(sH, LDN);
    }
    __syncthreads();

    // U_i = dy_i H_c: rows i (16 rw), columns n (64 cw)
    {
      f4 u[4];
      zero(u);
      if constexpr (BF)
        wave_gemm<BF, true, true, 4>(u, sDy + 16 * rw * LDP, LDP, 1, sH + 64 * cw * LDP, LDP, 1, Kp);
      else
        wave_gemm<BF, true, false, 4>(u, sDy + 16 * rw * LDP, LDP, 1, sH + 64 * cw, 1, LDN, Kp);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int il = 16 * rw + 4 * q + e, iq = i0 + il;
        const float ex = (iq < Q) ? __expf(sS[iq]) : 0.f;
        float part = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          part += u[t][e] * Op<BF>::back(sC[il * LDN + 64 * cw + 16 * t + r]);
          dca[t][e] += ex * u[t][e];
        }
        part = sum16(part);
        if (r == 0) sDso[cw][il] = part;
      }
    }

    float racc[2] = {0.f, 0.f};  // row sums for the lane's columns i
    for (int sl = 0; sl < nsl; ++sl) {
      const int s0 = sl * JW;
      __syncthreads();  // previous slab's reads of sXr done (and U's reads of sH)
      tXs.store(sXr, LDP);
      if (sl + 1 < nsl)
        tXs.load(x + (row0 + s0 + JW) * HP + static_cast<int64_t>(h) * P, HP, min(JW, jend - s0 - JW), P);
      else if (hh + 1 < hps)
        load_head(hh + 1);
      __syncthreads();
      float si[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) si[t] = sS[min(i0 + 32 * cw + 16 * t + r, Q - 1)];
#pragma unroll
      for (int jb = 0; jb < NBMAX; ++jb) {
        const int jl = jb * BQ - s0;
        if (jb <= ib && jl >= 0 && jl < JW) {
          // yx^T = x_j . dy_i: rows j, columns i
          f4 yx[2];
          zero(yx);
          wave_gemm<BF, true, true, 2>(yx, sXr + (jl + 16 * rw) * LDP, LDP, 1, sDy + 32 * cw * LDP, LDP, 1, Kp);
          float4* wsp = reinterpret_cast<float4*>(sWs + (jb * NT8 + tid) * 8);
          f4 ws[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if constexpr (BF) {
              const float4 v4 = wsp[t];
              ws[t] = f4{v4.x, v4.y, v4.z, v4.w};
            } else {
              ws[t] = wsr[jb][t];
            }
          }
          // the lane index taken here: masks and offsets built from it once
          // for the whole head loop would be spilled (one lane mask per
          // (block, tile, element))
          const int lo = opaque_index(lane_id()), ro = lo & 15, qo = lo >> 4;
          float sjv[4], dtjv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int jq = min(jb * BQ + 16 * rw + 4 * qo + e, Q - 1);
            sjv[e] = sS[jq];
            dtjv[e] = sDt[jq];
          }
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int iq = i0 + 32 * cw + 16 * t + ro, jq = jb * BQ + 16 * rw + 4 * qo + e;
              const bool valid = iq < Q && jq <= iq;
              const float ly = valid ? __expf(si[t] - sjv[e]) * yx[t][e] * dtjv[e] : 0.f;
              ws[t][e] += ly;
              if (jq < iq) racc[t] += ly * cb[jb][t][e];
            }
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if constexpr (BF)
              wsp[t] = make_float4(ws[t][0], ws[t][1], ws[t][2], ws[t][3]);
            else
              wsr[jb][t] = ws[t];
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float rr = sum_q(racc[t]);
      if (q == 0) sRow[rw][32 * cw + 16 * t + r] = rr;
    }
    // dD partial over this block's rows
    // (lane p of a 64-lane row group, rows il = tid / 64, +8, ...: no per-element division)
    float dd = 0.f;
    {
      const int p = tid % PMAX;
      if constexpr (!BF) {
        // f32 operands: this block's dy rows (sDy) and x rows (the last x
        // slab, JW = BQ rows from i0) are both still in LDS
        static_assert(BF || JW == BQ, "one block per f32 slab");
        if (p < P)
          for (int il = tid / PMAX; il < vi; il += NT8 / PMAX) dd += sDy[il * LDP + p] * sXr[il * LDP + p];
      } else {
        // (the staged dy is rounded to bf16 here: the products take dy as given)
        if (p < P)
          for (int il = tid / PMAX; il < vi; il += NT8 / PMAX) {
            const int64_t o = (row0 + i0 + il) * HP + static_cast<int64_t>(h) * P + p;
            dd += load_f(dy, o) * load_f(x, o);
          }
      }
    }
    dd = wave_sum(dd);
    if (l == 0) sTmp[8 + w] = dd;
    __syncthreads();
    if (tid < BQ && i0 + tid < Q) {
      const int64_t o = (static_cast<int64_t>(bi) * H + h) * T + static_cast<int64_t>(c) * Q + i0 + tid;
      rowM[o] = sRow[0][tid] + sRow[1][tid] + sRow[2][tid] + sRow[3][tid];
      dsoff[o] = __expf(sS[i0 + tid]) * (sDso[0][tid] + sDso[1][tid]);
    }
    if (tid == 0) {
      float tot = 0.f;
      for (int k = 0; k < NT8 / WAVE; ++k) tot += sTmp[8 + k];
      dD_part[((static_cast<int64_t>(bi) * nc + c) * nb + ib) * H + h] = tot;
    }
  }

  // dC_i += sum_j W[i][j] B_j with W = sum over heads of L yx dt
  for (int sl = 0; sl < nsl; ++sl) {
    const int s0 = sl * JW;
    __syncthreads();
#pragma unroll
    for (int jb = 0; jb < NBMAX; ++jb) {
      const int jl = jb * BQ - s0;
      if (jb <= ib && jl >= 0 && jl < JW) {
        const float4* wsp = reinterpret_cast<const float4*>(sWs + (jb * NT8 + tid) * 8);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float4 v4;
          if constexpr (BF)
            v4 = wsp[t];
          else
            v4 = make_float4(wsr[jb][t][0], wsr[jb][t][1], wsr[jb][t][2], wsr[jb][t][3]);
          OT* wp = sW + (32 * cw + 16 * t + r) * LDJ + jl + 16 * rw + 4 * q;
          if constexpr (BF)
            *reinterpret_cast<uint2*>(wp) = make_uint2(pack_bf16(v4.x, v4.y), pack_bf16(v4.z, v4.w));
          else
            *reinterpret_cast<float4*>(wp) = v4;
        }
      }
    }
    const int vj = min(JW, jend - s0);
    const TI* bsrc = Bm + (row0 + s0) * GN + static_cast<int64_t>(g) * N;
    if constexpr (BF) {
      TransTile<TI, JW, NMAX, 4, NT8> tb;
      tb.load(bsrc, GN, vj, N);
      tb.store(sBf, LDJ);
    } else {
      RowTile<TI, JW, NMAX, NT8> tb;
      tb.load(bsrc, GN, vj, N);
      tb.store(sBf, LDN);
    }
    __syncthreads();
    const int kw = round_up(vj, Op<BF>::KS);
    if constexpr (BF)
      wave_gemm<BF, true, true, 4>(dca, sW + 16 * rw * LDJ, LDJ, 1, sBf + 64 * cw * LDJ, LDJ, 1, kw);
    else
      wave_gemm<BF, true, false, 4>(dca, sW + 16 * rw * LDJ, LDJ, 1, sBf + 64 * cw, 1, LDN, kw);
  }
  const int64_t batch = gridDim.x / (nunit * nsplit * G * nc);
  float* dCo = dC_out + static_cast<int64_t>(sp) * batch * T * GN;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int iq = i0 + 16 * rw + 4 * q + e, n = 64 * cw + 16 * t + r;
      if (iq < Q && n < N) dCo[(row0 + iq) * GN + static_cast<int64_t>(g) * N + n] = dca[t][e];
    }
  }  // pass
}

// ------------------------------------------------------------- dt finalize
//
// ddt, and the dA_log and dD sums.  A workgroup takes one chunk of one batch
// row and up to NH heads, one wave per head (lane l holds the chunk's
// rows l + 64 e, so a chunk's scan and sums need no barrier).  dt and ddt
// ([b, T, H]) pass through LDS, so that their global accesses run along the
// heads.  Each wave leaves its head's dA partial for the chunk; the workgroup
// that finishes last (by a device-scope counter, which the row kernel of the
// same call zeroes) sums every head's partials in a fixed order, so the sums do
// not depend on which workgroup that is.  NH (16, 8 or 4 heads per
// workgroup) is the widest that still gives a grid of 64 workgroups.  In the
// final sums each thread adds one head's partials over a strided slice of the
// chunks, and one thread per head adds the slices in slice order.
//
// Ordering of the partials and the counter, without a release fence (which
// on gfx950 writes back every dirty line of the L2 in every workgroup:
// measured 42 us for this kernel instead of 10): the partials are agent-scope
// atomic stores, which gfx950 performs at the device's coherence point
// (written through the L2, not kept as dirty lines in one XCD's cache);
// s_waitcnt vmcnt(0) returns only after each of the wave's stores has been
// acknowledged there; the barrier after it orders every wave's wait before
// the one thread's counter increment (an agent-scope atomic, also performed at
// the coherence point).  The workgroup that sees the final count then issues
// an agent-scope acquire fence (it invalidates its non-coherent cache lines)
// and reads the partials with agent-scope atomic loads, which also go to the
// coherence point.  So every partial is in place before the count that
// selects the reader, and the reader fetches it from there.

// Lane 63's value, in every lane.
__device__ __forceinline__ float lane63(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), WAVE - 1));
}
// Sum over the 64 lanes of a wave, in every lane (DPP scan, then lane 63).
__device__ __forceinline__ float wave_total(float v) { return lane63(wave_scan(v)); }

template <typename TI, int NH>
__global__ __launch_bounds__(NH* WAVE) void bwd_dt_kernel(const TI* __restrict__ dt,
                                                               const float* __restrict__ A_log,
                                                               float* __restrict__ ddt, float* __restrict__ dA_log,
                                                               float* __restrict__ dD, BwdScratch s, int T, int H,
                                                               int Q, int npb, int nc, int nb) {
  constexpr int NTH = NH * WAVE;
  __shared__ float sT[QMAX][NH + 1];  // dt in, then ddt out: [row][head]
  __shared__ float sRed[2][NTH];      // the final sums' slice partials
  __shared__ int sFinal;
  const int u = blockIdx.x;  // chunk index bi * nc + c
  const int hg0 = blockIdx.y * NH;
  const int nh = min(NH, H - hg0);
  const int bi = u / nc, c = u - bi * nc;
  const int64_t r0 = static_cast<int64_t>(bi) * T + static_cast<int64_t>(c) * Q;  // the chunk's first row
  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  // this wave's head: the per-row sums are loaded first, so that their
  // latency overlaps the dt staging
  const int h = hg0 + min(w, nh - 1);
  const int64_t o0 = (static_cast<int64_t>(bi) * H + h) * T + static_cast<int64_t>(c) * Q;
  float cE[4], rP[4], rM[4], dE[4], dS[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int k = 64 * e + l;
    cE[e] = rP[e] = rM[e] = dE[e] = dS[e] = 0.f;
    if (k < Q && w < nh) {
      cE[e] = s.colE[o0 + k];
      rP[e] = s.Rp[o0 + k];
      if (s.row_slots == 0) {
        rM[e] = s.rowM[o0 + k];
      } else {
        // the slots of the 64-column blocks at or before row k's block, in order
        for (int jb = 0; jb <= (k >> 6) && jb < s.row_slots; ++jb) rM[e] += s.rowM[jb * s.slot_elems + o0 + k];
      }
      dE[e] = s.diagE[o0 + k];
      dS[e] = s.dsoff[o0 + k];
    }
  }
  const float ghl = (l < npb && w < nh) ? s.gh_part[(static_cast<int64_t>(u) * H + h) * npb + l] : 0.f;
  for (int i = tid; i < Q * NH; i += NTH) {
    const int k = i / NH, j = i % NH;
    sT[k][j] = j < nh ? load_f(dt, (r0 + k) * H + hg0 + j) : 0.f;
  }
  __syncthreads();
  if (w < nh) {
    const float A = -__expf(A_log[h]);
    float dv[4], ds[4];
    float sl = 0.f, tr = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = 64 * e + l;
      dv[e] = k < Q ? sT[k][w] : 0.f;
      ds[e] = rM[e] - dv[e] * (cE[e] - dE[e]) + dS[e] - dv[e] * rP[e];
      sl += dv[e] * A;
      tr += dv[e] * rP[e];
    }
    sl = wave_total(sl);  // s at the chunk's last row
    tr = wave_total(tr);
    const float gh = wave_total(ghl);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (64 * e + l == Q - 1) ds[e] += tr + __expf(sl) * gh;
    // da_k = sum of ds over rows k' >= k: the chunk total less the inclusive
    // prefix, plus ds_k
    float incl[4], carry = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float sc = wave_scan(ds[e]);
      incl[e] = carry + sc;
      carry += lane63(sc);
    }
    float pa = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = 64 * e + l;
      const float da = carry - incl[e] + ds[e];
      if (k < Q) sT[k][w] = cE[e] + rP[e] + A * da;
      pa += dv[e] * da;
    }
    pa = wave_total(pa);
    if (l == 0)
      __hip_atomic_store(s.dA_part + static_cast<int64_t>(u) * H + h, pa, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  for (int i = tid; i < Q * NH; i += NTH) {
    const int k = i / NH, j = i % NH;
    if (j < nh) ddt[(r0 + k) * H + hg0 + j] = sT[k][j];
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores, the dA partial among them, are complete
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(s.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sFinal = prev + 1 == gridDim.x * gridDim.y;
  }
  __syncthreads();
  if (!sFinal) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  // the last workgroup: thread tid adds head h0 + tid % hb over the chunks
  // tid / hb, tid / hb + np, ...; then one thread per head adds the np slices
  const int nbc = gridDim.x;
  for (int h0 = 0; h0 < H; h0 += NTH) {
    const int hb = min(NTH, H - h0), np = NTH / hb;
    const int hh = tid % hb, part = tid / hb;
    float a = 0.f, dd = 0.f;
    if (part < np) {
#pragma unroll 4
      for (int v = part; v < nbc; v += np) {
        a += __hip_atomic_load(s.dA_part + static_cast<int64_t>(v) * H + h0 + hh, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        for (int ib = 0; ib < nb; ++ib) dd += s.dD_part[(static_cast<int64_t>(v) * nb + ib) * H + h0 + hh];
      }
    }
    sRed[0][tid] = a;
    sRed[1][tid] = dd;
    __syncthreads();
    if (tid < hb) {
      float ta = 0.f, td = 0.f;
      for (int p = 0; p < np; ++p) {
        ta += sRed[0][p * hb + tid];
        td += sRed[1][p * hb + tid];
      }
      dA_log[h0 + tid] = -__expf(A_log[h0 + tid]) * ta;
      dD[h0 + tid] = td;
    }
    __syncthreads();
  }
}

// out = sum over sp of part[sp] (sp in order), for dB (blockIdx.y = 0) and dC
// (1) in one launch.  With n a multiple of 4 a thread takes four consecutive
// floats (every split's partial then starts 16-byte aligned: the partials
// start at 256-byte workspace offsets, the outputs are checked at the
// boundary); otherwise one float.
__global__ void split_sum_kernel(const float* __restrict__ partB, float* __restrict__ outB,
                                 const float* __restrict__ partC, float* __restrict__ outC, int64_t n, int nsplit) {
  const float* part = blockIdx.y ? partC : partB;
  float* out = blockIdx.y ? outC : outB;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if ((n & 3) == 0) {
    if (i >= (n >> 2)) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sp = 0; sp < nsplit; ++sp) {
      const float4 v = reinterpret_cast<const float4*>(part + static_cast<int64_t>(sp) * n)[i];
      acc.x += v.x, acc.y += v.y, acc.z += v.z, acc.w += v.w;
    }
    reinterpret_cast<float4*>(out)[i] = acc;
  } else {
    if (i >= n) return;
    float acc = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) acc += part[static_cast<int64_t>(sp) * n + i];
    out[i] = acc;
  }
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

static int64_t nblocks_chunk(const Dims& d, int nsplit, bool paired) {
  return static_cast<int64_t>(d.b) * d.nc() * d.G * nsplit * (paired ? (d.nb() + 1) / 2 : d.nb());
}

template <typename TI, typename TY, bool BF>
static void col_launch(const Dims& d, int nsplit, bool paired, const void* x, const void* B, const void* C, const void* dt,
                       const void* dy, const float* A_log, const float* D, const void* gamma, float* dx,
                       float* dB_out, const BwdScratch& s, hipStream_t st) {
  hipLaunchKernelGGL((paired ? chunk_bwd_col_kernel<TI, TY, BF, true> : chunk_bwd_col_kernel<TI, TY, BF, false>),
                     dim3(nblocks_chunk(d, nsplit, paired)), dim3(NT8), 0, st,
                     static_cast<const TI*>(x), static_cast<const TI*>(B), static_cast<const TI*>(C),
                     static_cast<const TI*>(dt), static_cast<const TY*>(dy), A_log, D,
                     static_cast<const typename Op<BF>::T*>(gamma), dx, dB_out, s.colE,
                     s.diagE, s.Rp, d.T, d.H, d.P, d.N, d.G, d.Q, nsplit);
}

hipError_t launch_chunk_bwd_col(const Dims& d, DType act, DType dyt, int nsplit, bool paired, const void* x,
                                const void* B, const void* C, const void* dt, const void* dy,
                                const float* A_log, const float* D, const void* gamma, float* dx,
                                float* dB_out, const BwdScratch& s, hipStream_t st) {
  if (act == BF16) {
    if (dyt == BF16)
      col_launch<uint16_t, uint16_t, true>(d, nsplit, paired, x, B, C, dt, dy, A_log, D, gamma, dx, dB_out, s, st);
    else
      col_launch<uint16_t, float, true>(d, nsplit, paired, x, B, C, dt, dy, A_log, D, gamma, dx, dB_out, s, st);
  } else {
    if (dyt == BF16)
      col_launch<float, uint16_t, false>(d, nsplit, paired, x, B, C, dt, dy, A_log, D, gamma, dx, dB_out, s, st);
    else
      col_launch<float, float, false>(d, nsplit, paired, x, B, C, dt, dy, A_log, D, gamma, dx, dB_out, s, st);
  }
  return hipGetLastError();
}

template <typename TI, typename TY, bool BF>
static void row_launch(const Dims& d, int nsplit, bool paired, const void* x, const void* B, const void* C, const void* dt,
                       const void* dy, const float* A_log, const float* states, float* dC_out, const BwdScratch& s,
                       hipStream_t st) {
  hipLaunchKernelGGL((paired ? chunk_bwd_row_kernel<TI, TY, BF, true> : chunk_bwd_row_kernel<TI, TY, BF, false>),
                     dim3(nblocks_chunk(d, nsplit, paired)), dim3(NT8), 0, st,
                     static_cast<const TI*>(x), static_cast<const TI*>(B), static_cast<const TI*>(C),
                     static_cast<const TI*>(dt), static_cast<const TY*>(dy), A_log, states, dC_out, s.rowM, s.dsoff,
                     s.dD_part, s.done, d.T, d.H, d.P, d.N, d.G, d.Q, nsplit);
}

hipError_t launch_chunk_bwd_row(const Dims& d, DType act, DType dyt, int nsplit, bool paired, const void* x,
                                const void* B, const void* C, const void* dt, const void* dy,
                                const float* A_log, const float* states, float* dC_out,
                                const BwdScratch& s, hipStream_t st) {
  if (act == BF16) {
    if (dyt == BF16)
      row_launch<uint16_t, uint16_t, true>(d, nsplit, paired, x, B, C, dt, dy, A_log, states, dC_out, s, st);
    else
      row_launch<uint16_t, float, true>(d, nsplit, paired, x, B, C, dt, dy, A_log, states, dC_out, s, st);
  } else {
    if (dyt == BF16)
      row_launch<float, uint16_t, false>(d, nsplit, paired, x, B, C, dt, dy, A_log, states, dC_out, s, st);
    else
      row_launch<float, float, false>(d, nsplit, paired, x, B, C, dt, dy, A_log, states, dC_out, s, st);
  }
  return hipGetLastError();
}

// Fewest workgroups per call.  The kernel is short and latency-bound: a grid
// of one workgroup per CU (4 heads each) measured slower than 64 workgroups of
// 16 heads (every workgroup stages its rows and adds itself to the arrival
// counter), while a grid of fewer than 64 gains from narrower workgroups.
constexpr int64_t DT_GRID_TARGET = 64;

template <typename TI, int NH>
static void dt_launch(const Dims& d, const void* dt, const float* A_log, float* ddt, float* dA_log, float* dD,
                      const BwdScratch& s, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(d.b) * d.nc()), (d.H + NH - 1) / NH);
  hipLaunchKernelGGL((bwd_dt_kernel<TI, NH>), grid, dim3(NH * WAVE), 0, st, static_cast<const TI*>(dt), A_log, ddt,
                     dA_log, dD, s, d.T, d.H, d.Q, state_npb(d), d.nc(), d.nb());
}

template <typename TI>
static void dt_dispatch(const Dims& d, const void* dt, const float* A_log, float* ddt, float* dA_log, float* dD,
                        const BwdScratch& s, hipStream_t st) {
  // the widest workgroup that still gives DT_GRID_TARGET workgroups
  const int64_t units = static_cast<int64_t>(d.b) * d.nc();
  if (units * ((d.H + 15) / 16) >= DT_GRID_TARGET)
    dt_launch<TI, 16>(d, dt, A_log, ddt, dA_log, dD, s, st);
  else if (units * ((d.H + 7) / 8) >= DT_GRID_TARGET)
    dt_launch<TI, 8>(d, dt, A_log, ddt, dA_log, dD, s, st);
  else
    dt_launch<TI, 4>(d, dt, A_log, ddt, dA_log, dD, s, st);
}

hipError_t launch_bwd_dt(const Dims& d, DType act, const void* dt, const float* A_log, float* ddt, float* dA_log,
                         float* dD, const BwdScratch& s, hipStream_t st) {
  if (act == BF16)
    dt_dispatch<uint16_t>(d, dt, A_log, ddt, dA_log, dD, s, st);
  else
    dt_dispatch<float>(d, dt, A_log, ddt, dA_log, dD, s, st);
  return hipGetLastError();
}

hipError_t launch_bwd_split_sum(const Dims& d, int nsplit, float* dB, float* dC, const BwdScratch& s,
                                hipStream_t st) {
  if (nsplit == 1) return hipSuccess;
  const int64_t n = static_cast<int64_t>(d.b) * d.T * d.G * d.N;
  const int64_t blocks = (((n & 3) == 0 ? n >> 2 : n) + 255) / 256;
  hipLaunchKernelGGL(split_sum_kernel, dim3(static_cast<unsigned>(blocks), 2), dim3(256), 0, st, s.dB_part, dB,
                     s.dC_part, dC, n, nsplit);
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
