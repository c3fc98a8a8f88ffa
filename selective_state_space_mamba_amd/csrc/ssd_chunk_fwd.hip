// Chunk output of the SSD forward.
//
// Inside one chunk (s_i = within-chunk inclusive cumsum of dt A, H_c the state
// entering the chunk) the recurrence of the reference page
// (burn_dragon_kernel src/sequence/mamba2/backward.rs, ssd_forward_state_history_reference,
// with the y readout of the block backward: y = sum_n ssm C + D x) is
//
//   y_i = sum_{j<=i} exp(s_i - s_j) (C_i . B_j) dt_j x_j     (intra-chunk part)
//       + exp(s_i) C_i . H_c^T                                (incoming state)
//       + D x_i.
//
// A workgroup owns one 64-row block ib of chunk c for a run of heads of one
// group.  It computes the group's (C.B^T)^T = B.C^T tiles (jb <= ib, ib) once
// with MFMA (K = d_state) and keeps them in registers (transposed, so that each
// lane's four values of the masked matrix are adjacent in LDS), then per head applies the decay
// mask L_ij = exp(s_i - s_j) (i >= j; exponents are <= 0) and dt_j, and runs
// the two remaining contractions (K = chunk columns, K = d_state) on MFMA.
// Operands are staged with 16-byte loads; the next head's x and H_c are loaded
// into registers while the current head computes.  bf16 operands stage the
// whole chunk width at once (one slab); f32 operands go 64 columns at a time.
// 8 waves: wave (rw, cw) = (w % 4, w / 4) owns rows 16*rw..+15 and columns
// 32*cw..+31 of every 64 x 64 tile, so two waves share each SIMD.
#include "ssd_async.hpp"
#include "ssd_common.hpp"
#include "ssd_launch.hpp"

namespace ssd {

template <bool BF> struct OutSlab { static constexpr int JW = BF ? QMAX : BQ; };

constexpr int NT8 = 512;

template <typename TI, bool BF>
__global__ __launch_bounds__(NT8) void chunk_out_fwd_kernel(
    const TI* __restrict__ x, const TI* __restrict__ Bm, const TI* __restrict__ Cm,
    const TI* __restrict__ dt, const float* __restrict__ A_log, const float* __restrict__ D,
    const float* __restrict__ hstates, TI* __restrict__ y, int T, int H, int P, int N, int G, int Q,
    int nsplit, int paired) {
  typedef typename Op<BF>::T OT;
  constexpr int PAD = BF ? 8 : 4;
  constexpr int JW = OutSlab<BF>::JW;  // chunk columns staged per slab
  constexpr int LDN = NMAX + PAD;      // [row][n]
  constexpr int LDJ = JW + PAD;        // [row][j]
  constexpr int PH1 = JW * LDN;                     // phase 1: B rows
  constexpr int PH2 = PMAX * LDN + PMAX * LDJ + BQ * LDJ;  // phase 2: H, x^T, G
  __shared__ __attribute__((aligned(16))) OT sC[BQ * LDN];
  __shared__ __attribute__((aligned(16))) OT sU[PH1 > PH2 ? PH1 : PH2];
  __shared__ float sS[QMAX];
  __shared__ float sDt[QMAX];
  __shared__ float sTmp[16];
  OT* const sB = sU;
  OT* const sH = sU;
  OT* const sXt = sU + PMAX * LDN;
  OT* const sG = sXt + PMAX * LDJ;

  const int nc = T / Q, nb = (Q + BQ - 1) / BQ;
  const int hpg = H / G, hps = hpg / nsplit;
  // paired: row blocks nb - 1 - k and then k, so that every workgroup has the
  // same number of (row block, column block) tiles; else one block, the
  // heavier ones first
  const int nunit = paired ? (nb + 1) >> 1 : nb;
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
  (void)l;
  const int64_t row0 = static_cast<int64_t>(bi) * T + static_cast<int64_t>(c) * Q;
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
  const int ib = pass ? unit : nb - 1 - unit;
  if (pass && (!paired || ib == nb - 1 - unit)) break;
  if (pass) __syncthreads();  // the first block's last head is done with sC and sU
  // the lane indices taken afresh in each pass: offsets derived from them
  // would otherwise be hoisted out of the pass loop and held across it
  const int r = opaque_index(lane_id()) & 15, q = opaque_index(lane_id()) >> 4;
  const int i0 = ib * BQ;
  const int vi = min(BQ, Q - i0);
  const int jend = min(Q, i0 + BQ);  // columns j < jend are needed
  const int nslab = (jend + JW - 1) / JW;
  const int Kn = round_up(N, Op<BF>::KS);
  const int64_t GN = static_cast<int64_t>(G) * N, HP = static_cast<int64_t>(H) * P;
  const int64_t PN = static_cast<int64_t>(P) * N;

  // ---- group-level C.B^T tiles for (ib, jb <= ib)
  {
    RowTile<TI, BQ, NMAX, NT8> tc;
    tc.load(Cm + (row0 + i0) * GN + static_cast<int64_t>(g) * N, GN, vi, N);
    tc.store(sC, LDN);
  }
  f4 cb[NBMAX][2];
#pragma unroll
  for (int jb = 0; jb < NBMAX; ++jb) zero(cb[jb]);
  for (int sl = 0; sl < nslab; ++sl) {
    const int j0 = sl * JW;
    RowTile<TI, JW, NMAX, NT8> tb;
    tb.load(Bm + (row0 + j0) * GN + static_cast<int64_t>(g) * N, GN, min(JW, jend - j0), N);
    __syncthreads();
    tb.store(sB, LDN);
    __syncthreads();
#pragma unroll
    for (int jb = 0; jb < NBMAX; ++jb) {
      const int jl = jb * BQ - j0;  // block start inside the slab
      if (jb <= ib && jl >= 0 && jl < JW)  // rows j of block jb (this wave's 16), columns i (its 32)
        wave_gemm<BF, true, true, 2>(cb[jb], sB + (jl + 16 * rw) * LDN, LDN, 1, sC + 32 * cw * LDN, LDN, 1, Kn);
    }
  }

  // ---- per head
  RowTile<float, PMAX, NMAX, NT8> th;      // H_c as [p][n]
  TransTile<TI, JW, PMAX, 4, NT8> tx;      // x rows j -> [p][j]
  float dt_next = 0.f;
  auto prefetch = [&](int hh, int sl) {
    const int h = g * hpg + sp * hps + hh;
    if (sl == 0) {
      th.load(hstates + ((static_cast<int64_t>(bi) * nc + c) * H + h) * PN, N, P, N);
      dt_next = (tid < Q) ? load_f(dt, (row0 + tid) * H + h) : 0.f;
    }
    const int j0 = sl * JW;
    tx.load(x + (row0 + j0) * HP + static_cast<int64_t>(h) * P, HP, min(JW, jend - j0), P);
  };
  prefetch(0, 0);

  for (int hh = 0; hh < hps; ++hh) {
    const int h = g * hpg + sp * hps + hh;
    const float A = -__expf(A_log[h]);
    const float Dh = D[h];
    const float dtv = dt_next;
    __syncthreads();  // the previous head is done with sS, sDt and the tiles
    const float s = block_inclusive_scan(dtv * A, sTmp);
    if (tid < Q) {
      sS[tid] = s;
      sDt[tid] = dtv;
    }
    th.store(sH, LDN);
    // skip term D x_i of this wave's output rows, loaded now, used at the end
    float xsk[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int iq = i0 + 16 * rw + 4 * q + i;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int p = 32 * cw + 16 * t + r;
        xsk[i][t] = (iq < Q && p < P) ? load_f(x, (row0 + iq) * HP + static_cast<int64_t>(h) * P + p) : 0.f;
      }
    }
    __syncthreads();

    // incoming-state readout: exp(s_i) * C_i . H_c^T
    f4 acc[2];
    zero(acc);
    wave_gemm<BF, true, true, 2>(acc, sC + 16 * rw * LDN, LDN, 1, sH + 32 * cw * LDN, LDN, 1, Kn);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int iq = i0 + 16 * rw + 4 * q + i;
      const float e = (iq < Q) ? __expf(sS[iq]) : 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) acc[t][i] *= e;
    }

    // intra-chunk part, one slab of chunk columns at a time
    for (int sl = 0; sl < nslab; ++sl) {
      const int j0 = sl * JW;
      if (sl > 0) __syncthreads();  // previous slab's MFMA reads done
      tx.store(sXt, LDJ);
#pragma unroll
      for (int jb = 0; jb < NBMAX; ++jb) {
        const int jl = jb * BQ - j0;
        if (jb <= ib && jl >= 0 && jl < JW) {
          // the lane index taken here: masks and offsets built from it once
          // for the whole head loop would be spilled
          const int lo = opaque_index(lane_id()), ro = lo & 15, qo = lo >> 4;
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            // lane holds B.C^T rows j = jb*64 + 16rw + 4q + e (e = 0..3), column i = i0 + 32cw + 16t + r
            const int il = 32 * cw + 16 * t + ro, iq = i0 + il;
            const int jw = 16 * rw + 4 * qo;  // first of the lane's four j inside block jb
            const float si = sS[min(iq, Q - 1)];
            float v4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int jq = jb * BQ + jw + e;
              const int jc = min(jq, Q - 1);
              v4[e] = (iq < Q && jq <= iq) ? cb[jb][t][e] * __expf(si - sS[jc]) * sDt[jc] : 0.f;
            }
            OT* gp = sG + il * LDJ + jl + jw;
            if constexpr (BF)
              *reinterpret_cast<uint2*>(gp) = make_uint2(pack_bf16(v4[0], v4[1]), pack_bf16(v4[2], v4[3]));
            else
              *reinterpret_cast<float4*>(gp) = make_float4(v4[0], v4[1], v4[2], v4[3]);
          }
        }
      }
      // next x slab (or the next head's first slab) loads while this one computes
      if (sl + 1 < nslab)
        prefetch(hh, sl + 1);
      else if (hh + 1 < hps)
        prefetch(hh + 1, 0);
      __syncthreads();
      const int kw = round_up(min(JW, jend - j0), Op<BF>::KS);
      wave_gemm<BF, true, true, 2>(acc, sG + 16 * rw * LDJ, LDJ, 1, sXt + 32 * cw * LDJ, LDJ, 1, kw);
    }

    // skip term and store
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int iq = i0 + 16 * rw + 4 * q + i, p = 32 * cw + 16 * t + r;
        if (iq < Q && p < P) {
          const int64_t o = (row0 + iq) * HP + static_cast<int64_t>(h) * P + p;
          store_f(y, o, acc[t][i] + Dh * xsk[i][t]);
        }
      }
  }
  }  // pass
}

hipError_t launch_chunk_out_fwd(const Dims& d, DType act, int nsplit, bool paired, const void* x, const void* B,
                                const void* C, const void* dt, const float* A_log, const float* D,
                                const float* states, void* y, hipStream_t st) {
  const int64_t nblk = static_cast<int64_t>(d.b) * d.nc() * d.G * nsplit * (paired ? (d.nb() + 1) / 2 : d.nb());
  if (act == BF16) {
    hipLaunchKernelGGL((chunk_out_fwd_kernel<uint16_t, true>), dim3(nblk), dim3(NT8), 0, st,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(B),
                       static_cast<const uint16_t*>(C), static_cast<const uint16_t*>(dt), A_log, D, states,
                       static_cast<uint16_t*>(y), d.T, d.H, d.P, d.N, d.G, d.Q, nsplit, paired ? 1 : 0);
  } else {
    hipLaunchKernelGGL((chunk_out_fwd_kernel<float, false>), dim3(nblk), dim3(NT8), 0, st,
                       static_cast<const float*>(x), static_cast<const float*>(B),
                       static_cast<const float*>(C), static_cast<const float*>(dt), A_log, D, states,
                       static_cast<float*>(y), d.T, d.H, d.P, d.N, d.G, d.Q, nsplit, paired ? 1 : 0);
  }
  return hipGetLastError();
}

}  // namespace ssd
