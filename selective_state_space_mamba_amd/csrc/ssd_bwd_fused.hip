// Intra-chunk backward of the SSD for bf16 operands in one kernel: the column
// work (dx, dB, column sums) and the row work (dC, row sums, readout term, dD)
// of one (batch, chunk, group) read x, dy, B, C, Gamma and H_c once.
//
// Formulas: those at the head of ssd_chunk_bwd.hip (derived there from the
// reverse-time loop of the reference page, burn_dragon_kernel
// src/sequence/mamba2/backward.rs, ssd_backward_reference).  With s the
// within-chunk cumsum of dt A, L_ij = exp(s_i - s_j), CB_ij = C_i . B_j and
// yx_ij = dy_i . x_j, the per-head matrices are G = L CB (dx), W = L yx dt_j
// (summed over heads: dB = W^T C, dC = W B) and M = W CB (row sums enter the
// decay gradient); U_i = dy_i H_c gives the readout term and the state part of
// dC.
//
// A workgroup owns one (batch, chunk, group) (or a run of the group's heads)
// and makes one pass per 64-column block jb of the chunk, in order.  Each pass
// is the column walk of ssd_bwd_bf16.hip (8 waves in two teams; a step is one
// head and one 64-row block ib >= jb: yx^T by MFMA, the decay terms, G to
// wave strips, dx_j += G^T dy on MFMA; per head the state terms with Gamma),
// and additionally:
//   * the strictly-lower row sums of M over the pass's 64 columns j, per step
//     (lanes, then the four waves of a team through LDS), stored to row-sum
//     slot jb (the dt kernel adds the slots jb <= ib of a row);
//   * on the diagonal step (ib = jb): the diagonal of yx (dD), and
//     U = dy_i H_c (MFMA, H_c in bf16 from LDS), the readout exp(s_i) U_i . C_i
//     and its head sum exp(s_i) U_i (the state part of dC for block jb);
//   * at the pass end: the head-summed W of the blocks below the diagonal
//     (ib > jb) to the workgroup's W area (bf16, one 8 KB block per pair
//     (ib, jb), read back by pass ib); dC of block jb, whole and stored once:
//     its state part plus sum_{j <= jb} W_{jb,j} B_j, the earlier passes' W
//     blocks copied from the W area and their B tiles kept in the C slots
//     those passes freed (C tile j is last read at the end of pass j); then
//     dB_j = sum_i W_ij C_i.
#include "ssd_async.hpp"
#include "ssd_common.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {
constexpr int FW = 8;               // waves per workgroup
constexpr int FT = FW * WAVE;       // threads per workgroup
constexpr int TILE_N = 64 * 256;    // bytes of a 64 x 128 bf16 tile
constexpr int TILE_P = 64 * 128;    // bytes of a 64 x 64 bf16 tile
constexpr int STRIP = 32 * 32;      // bytes of a 32 x 16 bf16 strip
constexpr int WPAIR_BYTES = FUSED_W_PAIR_BYTES;  // one 64 x 64 block of W in bf16
constexpr int KP = PMAX / 32;
constexpr int KN = NMAX / 32;
static_assert(NBMAX <= 4, "the pass-end phase holds at most four blocks' W strips");
static_assert(FUSED_GH_SLOTS == FW, "one <Gamma, H_c> partial per wave");

// Sum over the 64 lanes of a wave, in every lane (DPP scan, then lane 63).
__device__ __forceinline__ float lane_last(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), WAVE - 1));
}
__device__ __forceinline__ float wave_tot(float v) { return lane_last(wave_scan(v)); }

// A fragment of W (rows i, k = j) from the [i][j] wave strips of one block:
// rows i = 16 a + (lane % 16), columns j = 32 ks + 8 (lane / 16) .. +7.  Row i
// lies in the strips of team i / 32, column j in the strip of wave j / 16 of
// that team.
__device__ __forceinline__ bf16x8 w_rows_frag(const lds_char* strips, int a, int ks, int l = lane_id()) {
  const int r = l & 15, q = l >> 4;
  const int team = a >> 1, ri = 16 * (a & 1) + r;
  const lds_char* strip = strips + (4 * team + 2 * ks + (q >> 1)) * STRIP;
  return *(const __attribute__((address_space(3))) bf16x8*)(strip + strip_off(ri, 16 * (q & 1)));
}
}  // namespace

// FULL: headdim PMAX, d_state NMAX and chunk QMAX (every tile full), which
// lets the compiler drop the shape arguments and the row and column bounds
// checks; otherwise any shape bwd_bf16_supported accepts.
template <bool FULL>
__global__ __launch_bounds__(FT) void bwd_fused_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm,
    const uint16_t* __restrict__ dt, const uint16_t* __restrict__ dy, const float* __restrict__ A_log,
    const float* __restrict__ D, const uint16_t* __restrict__ gamma, const uint16_t* __restrict__ hbf,
    float* __restrict__ dx, float* __restrict__ dB_out, float* __restrict__ dC_out, float* __restrict__ ddt,
    float* __restrict__ dA_log_out, float* __restrict__ dD_out, BwdScratch s, int T, int H, int P_, int N_, int G,
    int Q_, int nsplit) {
  const int P = FULL ? PMAX : P_, N = FULL ? NMAX : N_, Q = FULL ? QMAX : Q_;
  __shared__ __attribute__((aligned(1024))) char sB_[TILE_N];          // B rows j of block jb
  __shared__ __attribute__((aligned(1024))) char sX_[2 * TILE_P];      // x rows j, two heads; W strip slot
  __shared__ __attribute__((aligned(1024))) char sDy0_[TILE_P];        // dy rows i, even steps
  __shared__ __attribute__((aligned(1024))) char sDy1_[TILE_P];        // dy rows i, odd steps; W strip slot
  __shared__ __attribute__((aligned(1024))) char sGam_[TILE_N];        // Gamma [p][n]; W strip slot
  __shared__ __attribute__((aligned(1024))) char sH_[TILE_N];          // H_c [p][n] (bf16)
  __shared__ __attribute__((aligned(1024))) char sG_[FW * STRIP];      // per-wave strips [i][j]; W strip slot
  // C tile of block ib at ib * 16 KB; after pass ib, B rows of block ib there
  __shared__ __attribute__((aligned(1024))) char sCt_[NBMAX * TILE_N];
  __shared__ float sRed[2][BQ][4];  // column sums, diagonal, R', readout: team halves
  __shared__ float sRm[4][BQ];      // one step's row sums of M per wave of a team; dD wave sums
  __shared__ float sDiag[BQ];       // the diagonal of E on the pass's diagonal block
  __shared__ __attribute__((aligned(16))) float sS[QMAX];
  __shared__ __attribute__((aligned(16))) float sDt[QMAX];
  __shared__ __attribute__((aligned(16))) uint32_t sDtb[QMAX];  // dt bits of the next head to scan
  lds_char* const sB = lds_ptr(sB_);
  lds_char* const sX = lds_ptr(sX_);
  lds_char* const sDy[2] = {lds_ptr(sDy0_), lds_ptr(sDy1_)};
  lds_char* const sGam = lds_ptr(sGam_);
  lds_char* const sH = lds_ptr(sH_);
  lds_char* const sG = lds_ptr(sG_);
  lds_char* const sCt = lds_ptr(sCt_);

  const int nc = T / Q, nb = (Q + BQ - 1) / BQ;
  const int hpg = H / G, hps = hpg / nsplit;
  int idx = xcd_logical_block(blockIdx.x, gridDim.x);
  const int sp = idx % nsplit;
  idx /= nsplit;
  const int g = idx % G;
  idx /= G;
  const int c = idx % nc;
  const int bi = idx / nc;
  const int64_t batch = gridDim.x / (static_cast<int64_t>(nsplit) * G * nc);

  const int l = lane_id(), w = wave_id(), r = l & 15, q = l >> 4;
  const int team = w >> 2, wt = w & 3;
  const int ti = 32 * team;  // this team's rows inside every 64-row block
  const RowsAt<8> r8_ = rows_at<8>();
  const RowsAt<16> r16_ = rows_at<16>();
  const ColsAt<2> c2_ = cols_at<2>();
  const ColsAt<8> c8_ = cols_at<8>();
  const ColsAt<16> c16_ = cols_at<16>();
  const AccAt<8> a8_ = acc_at<8>();
  const AccAt<16> a16_ = acc_at<16>();
  const int64_t row0 = static_cast<int64_t>(bi) * T + static_cast<int64_t>(c) * Q;
  const int64_t HP = static_cast<int64_t>(H) * P, GN = static_cast<int64_t>(G) * N;
  const uint32_t HPb = static_cast<uint32_t>(HP) * 2, GNb = static_cast<uint32_t>(GN) * 2;
  const uint32_t goff = static_cast<uint32_t>(g) * N * 2;
  const int pch = P >> 3, nch = N >> 3;
  const LazyRsrc rx{x + row0 * HP};
  const LazyRsrc rdy{dy + row0 * HP};
  const LazyRsrc rb{Bm + row0 * GN};
  const LazyRsrc rc{Cm + row0 * GN};
  const LazyRsrc rg{gamma + (static_cast<int64_t>(bi) * nc + c) * HP * N};
  const LazyRsrc rh{hbf + (static_cast<int64_t>(bi) * nc + c) * HP * N};
  const LazyRsrc rdx{dx + row0 * HP};
  // the per-head sums of (bi, h = 0, c): [b, H, T]
  const int64_t sum0 = static_cast<int64_t>(bi) * H * T + static_cast<int64_t>(c) * Q;
  const int64_t bht = batch * H * T;
  const LazyRsrc rcol{s.colE + sum0};
  const LazyRsrc rdiag{s.diagE + sum0};
  const LazyRsrc rrp{s.Rp + sum0};
  const LazyRsrc rdso{s.dsoff + sum0};
  // the per-wave partials of <Gamma_{c+1}, H_c> of (bi, c, h = 0)
  const LazyRsrc rgh{s.gh_part + (static_cast<int64_t>(bi) * nc + c) * H * FUSED_GH_SLOTS};
  // dB and dC (or this head split's partials) from the chunk's first row and the group's columns
  const LazyRsrc rdb{dB_out + static_cast<int64_t>(sp) * batch * T * GN + row0 * GN + static_cast<int64_t>(g) * N};
  const LazyRsrc rdc{dC_out + static_cast<int64_t>(sp) * batch * T * GN + row0 * GN + static_cast<int64_t>(g) * N};
  // this workgroup's W area: the head-summed W of its off-diagonal block pairs, bf16
  const int64_t wgi = ((static_cast<int64_t>(bi) * nc + c) * G + g) * nsplit + sp;
  const LazyRsrc rws{s.wstrips + wgi * (nb * (nb - 1) / 2) * (WPAIR_BYTES / 2)};

  // x and dy tiles (64 rows of headdim), Gamma and H_c (headdim rows of
  // d_state): per-lane offsets computed once, the tile's first row as the
  // scalar offset
  TileLanes<64, 8, FW> tl8;
  TileLanes<64, 16, FW> tlg;
  tl8.init(HPb, pch);
  tlg.init(N * 2, nch);

  // odd passes take the heads in reverse order, so that the tiles the
  // previous pass read last are still in L2
  auto head_of = [&](int jbp, int hh) { return g * hpg + sp * hps + ((jbp & 1) ? hps - 1 - hh : hh); };
  // the first tiles of pass jbp (the pass over column block jbp): the first
  // head's x (slot 0), dy on the diagonal block, H_c and dt; the B rows; the
  // first head's Gamma.  A pass
  // issues the next pass's tiles during its last phase, in that order (B once
  // the phase's last B reads are done, Gamma last: it is first read at the
  // first head's state step)
  auto load_first_xdhd = [&](int jbp) {
    const int h0 = head_of(jbp, 0), jx0 = jbp * BQ, vjx = min(BQ, Q - jx0);
    tl8.issue(sX, rx.get(), jx0 * HPb + h0 * P * 2, vjx);
    tl8.issue(sDy[0], rdy.get(), jx0 * HPb + h0 * P * 2, vjx);
    tlg.issue(sH, rh.get(), h0 * P * N * 2, P);
    steps_async<FW>(lds_ptr(sDtb), make_rsrc(dt + row0 * H + h0), H * 2, Q);
  };
  auto load_first_b = [&](int jbp) {
    const int jx0 = jbp * BQ;
    tile_async<64, 16, FW>(sB, rb.get(), jx0 * GNb + goff, GNb, min(BQ, Q - jx0), nch);
  };
  auto load_first_gam = [&](int jbp) { tlg.issue(sGam, rg.get(), head_of(jbp, 0) * P * N * 2, P); };

  // pass 0's first tiles and every block's C tile (later passes read a subset)
  load_first_xdhd(0);
  load_first_b(0);
#pragma unroll
  for (int u = 0; u < NBMAX; ++u) {
    if (u < nb) {
      const int i0 = u * BQ;
      tile_async<64, 16, FW>(sCt + u * TILE_N, rc.get(), i0 * GNb + goff, GNb, min(BQ, Q - i0), nch);
    }
  }
  load_first_gam(0);

  for (int jb = 0; jb < nb; ++jb) {
    auto head = [&](int hh) { return head_of(jb, hh); };
    const int j0 = jb * BQ, vj = min(BQ, Q - j0);
    const int nib = nb - jb;
    auto load_dt_abs = [&](int h) { steps_async<FW>(lds_ptr(sDtb), make_rsrc(dt + row0 * H + h), H * 2, Q); };
    auto load_x = [&](int hh) { tl8.issue(sX + (hh & 1) * TILE_P, rx.get(), j0 * HPb + head(hh) * P * 2, vj); };
    auto load_dy = [&](int hh, int u, lds_char* dst) {
      const int i0 = (jb + u) * BQ;
      tl8.issue(dst, rdy.get(), i0 * HPb + head(hh) * P * 2, min(BQ, Q - i0));
    };
    auto load_gam = [&](int hh) { tlg.issue(sGam, rg.get(), head(hh) * P * N * 2, P); };
    auto load_h = [&](int hh) { tlg.issue(sH, rh.get(), head(hh) * P * N * 2, P); };
    const __amdgpu_buffer_rsrc_t rrm = make_rsrc_ptr(s.rowM + static_cast<int64_t>(jb) * bht + sum0);

    // ---- the pass's first tiles (issued before the loop or during the
    // previous pass's last phase): all but the first head's Gamma must be in
    // LDS; then C.B^T for every block ib >= jb
    if (jb == 0)
      wait_vm<0>();
    else
      wait_vm<4>();  // the first head's Gamma and the previous pass's B tile (read at this pass's end) may be in flight
    lds_barrier();
    f4 cbk[NBMAX][2];  // C.B^T: rows j of this wave, columns i = (jb + u) * 64 + ti + 16 tt + r
#pragma unroll
    for (int u = 0; u < NBMAX; ++u) {
      zero(cbk[u]);
      if (u < nib) {
        bf16x8 bfr[KN];  // this wave's B rows j
        {
          const RowsAt<16> ar16 = opaque(r16_);
#pragma unroll
          for (int ks = 0; ks < KN; ++ks) bfr[ks] = frag_rows(sB, 16 * wt, 4 * ks, ar16);
        }
        const lds_char* ct = sCt + (jb + u) * TILE_N;
        const RowsAt<16> ar16 = opaque(r16_);
        bf16x8 fb[KN][2];
#pragma unroll
        for (int ks = 0; ks < KN; ++ks)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) fb[ks][tt] = frag_rows(ct, ti + 16 * tt, 4 * ks, ar16);
        sched_ds_reads<2 * KN>();
#pragma unroll
        for (int ks = 0; ks < KN; ++ks)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) cbk[u][tt] = mfma(bfr[ks], fb[ks][tt], cbk[u][tt]);
        sched_mfmas<2 * KN>();
      }
    }
    scan_store(sDtb, -__expf(A_log[head(0)]), sS, sDt);
    __syncthreads();

    f4 ws[NBMAX][2];  // sum over heads of L yx dt: rows j, columns i as in cbk
    f4 dbs[4];        // state part of dB: rows j, columns n = 16 (4 team + k) + r
    f4 ua[4];         // sum over heads of exp(s_i) U_i on the diagonal block: rows i = j0 + 16 wt + 4q + e,
                      // columns n = 16 (4 team + k) + r
#pragma unroll
    for (int u = 0; u < NBMAX; ++u) zero(ws[u]);
    zero(dbs);
    zero(ua);

    for (int hh = 0; hh < hps; ++hh) {
      const int h = head(hh), hb = hh & 1;
      const lds_char* xt = sX + hb * TILE_P;
      // s_j and dt_j of this lane's rows j = jq0 .. jq0 + 3, read where used
      // (entries past Q hold the chunk's last cumsum value and dt = 0; every
      // use at rows j >= Q is masked or multiplied by a zero operand)
      const int jq0 = j0 + 16 * wt + 4 * q;
      auto s_rows = [&](float (&v)[4]) {
        const float4 t = *reinterpret_cast<const float4*>(sS + opaque_index(jq0));
        v[0] = t.x, v[1] = t.y, v[2] = t.z, v[3] = t.w;
      };
      auto dt_rows = [&](float (&v)[4]) {
        const float4 t = *reinterpret_cast<const float4*>(sDt + opaque_index(jq0));
        v[0] = t.x, v[1] = t.y, v[2] = t.z, v[3] = t.w;
      };
      f4 dxa[2];  // sum over rows i of G_ij dy_i: rows j, columns p = 16 (2 team + k) + r
      zero(dxa);
      float Dh = 0.f, An = 0.f;
      float cfc[4], sprev = 0.f;
      float csum[4] = {0.f, 0.f, 0.f, 0.f};
      float ddv = 0.f;  // the diagonal of yx (dD)
      u32x2 dsk[2];     // dy_j at columns p = ti + 16 k + r, accumulator layout

#pragma unroll
      for (int u = 0; u < NBMAX; ++u) {
        if (u < nib) {
          const RowsAt<8> ar8 = opaque(r8_);
          const ColsAt<2> ac2 = opaque(c2_);
          const ColsAt<8> ac8 = opaque(c8_);
          const int i0 = (jb + u) * BQ;
          const lds_char* dyt = sDy[u & 1];
          // issue order of the step's copies: the next block's dy; at step 1
          // the next head's H_c (this head's was read in step 0); at step 0 the
          // next head's dt, last, so that the step's end need not wait for it
          if (u + 1 < nib) load_dy(hh, u + 1, sDy[(u + 1) & 1]);
          if (u == 1 && hh + 1 < hps) load_h(hh + 1);
          if (u == 0) {
            Dh = D[h];
            if (hh + 1 < hps) {
              An = A_log[head(hh + 1)];
              load_dt_abs(head(hh + 1));
            }
          }

          f4 yx[2];
          zero(yx);
          f4 cbt[2];
          float sv[2];
          float sref;
          const int ib0 = opaque_index(i0 + ti + r);
          {
            bf16x8 fb[KP][2], xf[KP];  // dy rows i; this wave's x rows j
#pragma unroll
            for (int ks = 0; ks < KP; ++ks) {
              xf[ks] = frag_rows(xt, 16 * wt, 4 * ks, ar8);
#pragma unroll
              for (int tt = 0; tt < 2; ++tt) fb[ks][tt] = frag_rows(dyt, ti + 16 * tt, 4 * ks, ar8);
            }
            cbt[0] = cbk[u][0];
            cbt[1] = cbk[u][1];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) sv[tt] = sS[min(ib0 + 16 * tt, Q - 1)];
            sref = sS[i0];
            sched_ds_reads<3 * KP + 3>();
#pragma unroll
            for (int ks = 0; ks < KP; ++ks)
#pragma unroll
              for (int tt = 0; tt < 2; ++tt) yx[tt] = mfma(xf[ks], fb[ks][tt], yx[tt]);
            sched_mfmas<2 * KP>();
          }
          f4 gv[2];
          float rmv[2] = {0.f, 0.f};  // row sums of M (rows i = i0 + ti + 16 tt + r) over this lane's 4 columns
          if (u == 0) {
            float sj[4], dtj[4];
            s_rows(sj);
            dt_rows(dtj);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
              const int iq = ib0 + 16 * tt;
              const float si = sv[tt];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int jq = opaque_index(jq0) + e;
                const float ex = __expf(si - sj[e]);
                const float L = (iq < Q && iq >= jq) ? ex : 0.f;
                const float G1 = L * cbt[tt][e];
                const float E = G1 * yx[tt][e];
                csum[e] += E;
                if (iq == jq) {
                  sDiag[jq - j0] = E;  // one lane of the workgroup holds each diagonal element
                  ddv += yx[tt][e];
                }
                const float Wv = L * dtj[e] * yx[tt][e];
                ws[u][tt][e] += Wv;
                if (jq < iq) rmv[tt] += Wv * cbt[tt][e];
                gv[tt][e] = G1;
              }
            }
            const AccAt<8> aa8 = opaque(a8_);
#pragma unroll
            for (int k = 0; k < 2; ++k) dsk[k] = block_acc(dyt, 16 * wt, ti + 16 * k, aa8);
          } else {
            float cf[4], cfd[4], dtj[4];
            dt_rows(dtj);
            if (u == 1) {
              float sj[4];
              s_rows(sj);
#pragma unroll
              for (int e = 0; e < 4; ++e) cfc[e] = __expf(sref - sj[e]);
            } else {
              const float adv = __expf(sref - sprev);
#pragma unroll
              for (int e = 0; e < 4; ++e) cfc[e] *= adv;
            }
            sprev = sref;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              cf[e] = cfc[e];
              cfd[e] = cf[e] * dtj[e];
            }
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
              const int iq = ib0 + 16 * tt;
              const float rx_ = __expf(sv[tt] - sref);
              const float rf = (iq < Q) ? rx_ : 0.f;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float G1 = rf * cf[e] * cbt[tt][e];
                const float E = G1 * yx[tt][e];
                csum[e] += E;
                const float Wv = rf * cfd[e] * yx[tt][e];
                ws[u][tt][e] += Wv;
                rmv[tt] += Wv * cbt[tt][e];
                gv[tt][e] = G1;
              }
            }
          }
          put_strip(sG + w * STRIP, gv);
          // this wave's row sums over its 16 columns (the 4 lane groups), to
          // LDS for the team sum
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) rmv[tt] = sum_q(rmv[tt]);
          if (q == 0) {
            sRm[wt][ti + r] = rmv[0];
            sRm[wt][ti + 16 + r] = rmv[1];
          }
          if (u == 0) {
            // U = dy_i H_c on the diagonal block: rows i = j0 + 16 wt + 4q + e,
            // columns n = 16 (4 team + k) + r; its readout exp(s_i) U_i . C_i
            // (team halves to LDS) and its head sum exp(s_i) U_i
            f4 uu[4];
            zero(uu);
            const RowsAt<8> ar8u = opaque(r8_);
            const ColsAt<16> ac16 = opaque(c16_);
#pragma unroll
            for (int ks = 0; ks < KP; ++ks) {
              const bf16x8 fa = frag_rows(dyt, 16 * wt, 4 * ks, ar8u);
              bf16x8 fb[4];
#pragma unroll
              for (int k = 0; k < 4; ++k) fb[k] = frag_cols(sH, 32 * ks, 16 * (4 * team + k), ac16);
              sched_ds_reads<9>();
#pragma unroll
              for (int k = 0; k < 4; ++k) uu[k] = mfma(fa, fb[k], uu[k]);
              sched_mfmas<4>();
            }
            const AccAt<16> aa16 = opaque(a16_);
            u32x2 ca[4];  // C_i at columns n = 16 (4 team + k) + r, accumulator layout
            const lds_char* ctd = sCt + jb * TILE_N;
#pragma unroll
            for (int k = 0; k < 4; ++k) ca[k] = block_acc(ctd, 16 * wt, 16 * (4 * team + k), aa16);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int il = 16 * wt + 4 * q + e;
              const float xe = __expf(sS[min(j0 + il, Q - 1)]);
              const float exi = (j0 + il < Q) ? xe : 0.f;
              float part = 0.f;
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                part += uu[k][e] * acc_elem(ca[k], e);
                ua[k][e] += exi * uu[k][e];
              }
              part = row_sum16(part);
              if (r == 15) sRed[team][il][3] = exi * part;
            }
          }
          lds_barrier();
          // dx_j += sum_i G_ij dy_i over the block's 64 rows i: k-step ks reads
          // the strip of team ks
          {
            bf16x8 ga[2], gb[2][2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              ga[ks] = frag_cols(sG + (4 * ks + wt) * STRIP, 0, 0, ac2);
#pragma unroll
              for (int k = 0; k < 2; ++k) gb[ks][k] = frag_cols(dyt, 32 * ks, 16 * (2 * team + k), ac8);
            }
            sched_ds_reads<12>();
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
              for (int k = 0; k < 2; ++k) dxa[k] = mfma(ga[ks], gb[ks][k], dxa[k]);
            sched_mfmas<4>();
          }
          // the step's row sums of M: wave 0 adds the four waves of each team
          // and stores them (row sum slot jb, rows i0 + l)
          if (w == 0) {
            const float rs = sRm[0][l] + sRm[1][l] + sRm[2][l] + sRm[3][l];
            const int il = i0 + opaque_index(l);  // recomputed here: hoisted per block it would stay live
            store_f32(rrm, rs, il < Q ? static_cast<uint32_t>(il) * 4 : OOB_OFFSET,
                      static_cast<uint32_t>(h) * T * 4);
          }
          // wave 0's row-sum store is its youngest memory operation; every
          // wave leaves the next head's dt copy in flight at step 0
          if (u == 0 && hh + 1 < hps) {
            if (w == 0)
              wait_vm<2>();
            else
              wait_vm<1>();
          } else {
            if (w == 0)
              wait_vm<1>();
            else
              wait_vm<0>();
          }
          lds_barrier();
          if (jb == 0 && u == 0) {
            // <Gamma_{c+1}, H_c> of head h, while both tiles are this head's
            // (Gamma has landed: this step's waits covered every copy issued
            // before it; H_c is replaced from step 1 or the state step on):
            // the two tiles share one layout, so matching 16-byte chunks hold
            // matching elements.  One partial per wave, added in wave order
            // by the dt epilogue.
            float gp = 0.f;
            const int tg = opaque_index(static_cast<int>(threadIdx.x));  // recomputed here: see the row-sum store
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const int off = (half * FT + tg) * 16;
              const bf16x8 ga = *(const __attribute__((address_space(3))) bf16x8*)(sGam + off);
              const bf16x8 ha = *(const __attribute__((address_space(3))) bf16x8*)(sH + off);
#pragma unroll
              for (int k = 0; k < 8; ++k) gp += static_cast<float>(ga[k]) * static_cast<float>(ha[k]);
            }
            gp = wave_tot(gp);
            store_f32(rgh.ptr(), gp, l == 0 ? 0u : OOB_OFFSET, static_cast<uint32_t>(h * FUSED_GH_SLOTS + w) * 4);
          }
        }
      }

      // ---- state terms of head hh; the next head's x and dy tiles start
      // loading (after its H_c when there was no step 1 to issue that), its
      // Gamma once this head's is read
      const RowsAt<16> ar16 = opaque(r16_);
      const ColsAt<16> ac16 = opaque(c16_);
      const bool h_here = nib == 1 && hh + 1 < hps;
      if (h_here) load_h(hh + 1);
      if (hh + 1 < hps) {
        load_x(hh + 1);
        load_dy(hh + 1, 0, sDy[0]);
      }
      f4 bg[2];  // B_j Gamma^T: rows j, columns p = 16 (2 team + k) + r
      zero(bg);
#pragma unroll
      for (int kh = 0; kh < KN; kh += 2) {
        bf16x8 fb[2][2], bfr[2];  // Gamma rows p; this wave's B rows j (from the pass's B tile)
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2) {
          bfr[d2] = frag_rows(sB, 16 * wt, 4 * (kh + d2), ar16);
#pragma unroll
          for (int k = 0; k < 2; ++k) fb[d2][k] = frag_rows(sGam, 16 * (2 * team + k), 4 * (kh + d2), ar16);
        }
        sched_ds_reads<6>();
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
          for (int k = 0; k < 2; ++k) bg[k] = mfma(bfr[d2], fb[d2][k], bg[k]);
        sched_mfmas<4>();
      }
      f4 v[4];  // x_j Gamma for this team's d_state columns
      zero(v);
      {
        const RowsAt<8> ar8 = opaque(r8_);
#pragma unroll
        for (int ks = 0; ks < KP; ++ks) {
          bf16x8 fb[4];
          const bf16x8 xf = frag_rows(xt, 16 * wt, 4 * ks, ar8);
#pragma unroll
          for (int k = 0; k < 4; ++k) fb[k] = frag_cols(sGam, 32 * ks, 16 * (4 * team + k), ac16);
          sched_ds_reads<9>();
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = mfma(xf, fb[k], v[k]);
          sched_mfmas<4>();
        }
      }
      u32x2 xa[2];
      {
        const AccAt<8> aa8 = opaque(a8_);
#pragma unroll
        for (int k = 0; k < 2; ++k) xa[k] = block_acc(xt, 16 * wt, 16 * (2 * team + k), aa8);
      }
      const float s_end = sS[Q - 1];
      float wj[4], dtj[4];
      {
        float sj[4];
        s_rows(sj);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float wx = __expf(s_end - sj[e]);
          wj[e] = (jq0 + e < Q) ? wx : 0.f;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int jl = 16 * wt + 4 * q + e;
        float part = 0.f;
#pragma unroll
        for (int k = 0; k < 2; ++k) part += bg[k][e] * acc_elem(xa[k], e);
        part = row_sum16(part);
        const float cs = row_sum16(csum[e]);
        if (r == 15) {
          sRed[team][jl][0] = cs;
          sRed[team][jl][2] = wj[e] * part;
        }
      }
      {
        const float dd = wave_sum(ddv);
        if (l == 0) sRm[0][w] = dd;
      }
      // dt_j before the barrier: the scan at this step's end overwrites it
      dt_rows(dtj);
      // the next head's dt copy must be in LDS; its H_c (when issued here), x
      // and dy copies may be in flight
      if (h_here)
        wait_vm<4>();
      else if (hh + 1 < hps)
        wait_vm<2>();
      lds_barrier();
      if (hh + 1 < hps) load_gam(hh + 1);  // this head's Gamma is no longer read
      float dxv[2][4];
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) dxv[k][e] = dtj[e] * (dxa[k][e] + wj[e] * bg[k][e]) + Dh * acc_elem(dsk[k], e);
      const int jc = 16 * wt + r;
      const float ce = sRed[0][jc][0] + sRed[1][jc][0];
      const float de = sDiag[jc];
      const float re = sRed[0][jc][2] + sRed[1][jc][2];
      const float so = sRed[0][jc][3] + sRed[1][jc][3];
      float dd_tot = 0.f;
      if (w == 0 && l == 0) {
#pragma unroll
        for (int k = 0; k < FW; ++k) dd_tot += sRm[0][k];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f = dtj[e] * wj[e];
#pragma unroll
        for (int k = 0; k < 4; ++k) dbs[k][e] += f * v[k][e];
      }
      // the next head's H_c, x and dy tiles (all but Gamma's 2 copies) must be
      // in LDS at the barrier; the stores below are issued after the wait and
      // complete during the next step
      if (hh + 1 < hps) wait_vm<2>();
      {
        const int lf = opaque_index(l), rf = lf & 15, qf = lf >> 4;  // recomputed: see the row-sum store
        const uint32_t vdx = (static_cast<uint32_t>(j0 + 16 * wt + 4 * qf) * HP + 32 * team + rf) * 4;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool ok = j0 + 16 * wt + 4 * qf + e < Q && 32 * team + 16 * k + rf < P;
            store_f32(rdx.ptr(), dxv[k][e], ok ? vdx + 64 * k : OOB_OFFSET, static_cast<uint32_t>(e * HP + h * P) * 4);
          }
        }
        if (team == 0) {
          const int jcf = 16 * wt + rf;
          const uint32_t vo = (qf == 0 && j0 + jcf < Q) ? static_cast<uint32_t>(j0 + jcf) * 4 : OOB_OFFSET;
          const uint32_t so4 = static_cast<uint32_t>(h) * T * 4;
          store_f32(rcol.ptr(), ce, vo, so4);
          store_f32(rdiag.ptr(), de, vo, so4);
          store_f32(rrp.ptr(), re, vo, so4);
          store_f32(rdso.ptr(), so, vo, so4);
        }
        // read by the last workgroup of this launch: stored at the device's coherence point
        if (w == 0 && l == 0)
          __hip_atomic_store(s.dD_part + ((static_cast<int64_t>(bi) * nc + c) * nb + jb) * H + h, dd_tot,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (hh + 1 < hps) scan_store(sDtb, -__expf(An), sS, sDt);
      lds_barrier();
    }

    // ---- pass end.  The W strips of blocks u = 0..3 go to four free 8 KB
    // slots; the strips of the blocks below the diagonal (ib > jb) also go to
    // the workgroup's W area in global memory, read back by pass ib.  dC of
    // the diagonal block is formed whole: its state part plus
    // sum_{j <= jb} W_{jb,j} B_j, k = j along the strips (this pass's) or the
    // W area (earlier passes'), against the B tile (j = jb) or the B tiles that
    // earlier passes left in the freed C slots (j < jb); then
    // dB_j = sum_i W_ij C_i + state terms over all rows i (k = i down the
    // strips, against the C tiles).  The next pass's first tiles load
    // meanwhile.
    // element (row0 + 4q + e, col0 + r) of a [rows][G N] f32 array (dB, dC)
    // at byte offset voff + soff: the lane's part voff (OOB_OFFSET outside
    // the chunk or d_state) and the uniform part soff
    const int lg = opaque_index(l), rg_ = lg & 15, qg = lg >> 4;  // recomputed: see the row-sum store
    const uint32_t gn_lane = (static_cast<uint32_t>(4 * qg) * static_cast<uint32_t>(GN) + rg_) * 4;
    auto gn_voff = [&](int row0_, int col0, int e) -> uint32_t {
      if (FULL) return gn_lane;
      return (row0_ + 4 * qg + e < Q && col0 + rg_ < N) ? gn_lane : OOB_OFFSET;
    };
    auto gn_soff = [&](int row0_, int col0, int e) -> uint32_t {
      return (static_cast<uint32_t>(row0_ + e) * static_cast<uint32_t>(GN) + col0) * 4;
    };
    // W fragments (rows i = 16 a + (lane % 16) of block ib, k = j = 32 ks +
    // 8 (lane / 16) .. + 7 of block j) in the W area: pair (ib, j), j < ib, at
    // WPAIR_BYTES (ib (ib - 1) / 2 + j), fragment (a, ks) at 1 KB (2 a + ks),
    // 16 bytes a lane.  This pass's pairs (jb, j < jb) are copied first, into
    // slots the strips below leave free (the Gamma tile's, then dy buffer 1)
    const uint32_t wlane = static_cast<uint32_t>(lg) * 16;
    auto wfrag_off = [&](int ib, int j, int a, int ks) -> uint32_t {
      return static_cast<uint32_t>((ib * (ib - 1) / 2 + j) * WPAIR_BYTES + (2 * a + ks) * 1024);
    };
    lds_char* const wprev[NBMAX - 1] = {sGam, sGam + WPAIR_BYTES, sDy[1]};
    static_assert(2 * WPAIR_BYTES <= TILE_N && WPAIR_BYTES <= TILE_P, "earlier W pairs fit the free slots");
    // (the wave index passes through an empty asm: copy addresses hoisted
    // out of the pass loop would hold registers for the whole kernel)
    int wo = w;
    asm volatile("" : "+s"(wo));
#pragma unroll
    for (int j = 0; j < NBMAX - 1; ++j)
      if (j < jb) dma16_so(rws.get(), wprev[j] + wo * 1024, wlane, wfrag_off(jb, j, 0, 0) + wo * 1024);
    // x slot 0, dy buffer 0, H_c and the dt bits are free (the last head's
    // state step is done; the strips below use the other slots)
    if (jb + 1 < nb) load_first_xdhd(jb + 1);
    lds_char* const wset[4] = {sG, sX + TILE_P, sDy[1], sGam};
#pragma unroll
    for (int u = 0; u < NBMAX; ++u)
      if (u < nib) put_strip(wset[u] + w * STRIP, ws[u]);
    // the earlier W pairs must be in LDS; the next pass's first tiles (5
    // copies) may be in flight
    if (jb > 0) {
      if (jb + 1 < nb)
        wait_vm<5>();
      else
        wait_vm<0>();
    }
    lds_barrier();
    // the strips of blocks ib = jb + u > jb to the W area: wave w stores
    // fragment (a, ks) = (w % 4, w / 4) of each.  Pass ib reads them after
    // the waits and barriers of the passes between (each of its waves waits
    // for every store it issued before the next pass's Gamma copy, then meets
    // the others at a barrier), from lines no earlier load of this launch
    // touched
#pragma unroll
    for (int u = 1; u < NBMAX; ++u) {
      if (u < nib) {
        // the lane passes through opaque_index: offsets hoisted out of the
        // pass loop would be spilled, and a spill's reload waits for every
        // copy in flight
        const bf16x8 fw = w_rows_frag(wset[u], wt, team, opaque_index(lane_id()));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, fw), rws.ptr(), wlane,
                                               wfrag_off(jb + u, jb, 0, 0) + (2 * (wo & 3) + (wo >> 2)) * 1024, 0);
      }
    }
    {
      // dC of block jb: rows i = 16 wt + 4q + e, columns n = 16 (4 team + k) + r
      const ColsAt<16> ac16 = opaque(c16_);
      f4 pc[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) pc[k] = ua[k];
#pragma unroll
      for (int j = 0; j < NBMAX; ++j) {
        if (j <= jb) {
          const lds_char* bt = j == jb ? sB : sCt + j * TILE_N;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            bf16x8 fa, fb[4];
            if (j == jb)
              fa = w_rows_frag(wset[0], wt, ks);
            else
              fa = *(const __attribute__((address_space(3))) bf16x8*)(wprev[j < NBMAX - 1 ? j : 0] +
                                                                       (2 * wt + ks) * 1024 + wlane);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) fb[kk] = frag_cols(bt, 32 * ks, 16 * (4 * team + kk), ac16);
            sched_ds_reads<5>();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) pc[kk] = mfma(fa, fb[kk], pc[kk]);
            sched_mfmas<4>();
          }
        }
      }
      const int r0 = j0 + 16 * wt;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c0 = 16 * (4 * team + k);
#pragma unroll
        for (int e = 0; e < 4; ++e) store_f32(rdc.ptr(), pc[k][e], gn_voff(r0, c0, e), gn_soff(r0, c0, e));
      }
    }
    lds_barrier();  // the B tile is no longer read
    if (jb + 1 < nb) load_first_b(jb + 1);
    f4 dbp[4];
    zero(dbp);
#pragma unroll
    for (int u = 0; u < NBMAX; ++u) {
      if (u < nib) {
        const lds_char* ct = sCt + (jb + u) * TILE_N;
        const ColsAt<2> ac2 = opaque(c2_);
        const ColsAt<16> ac16 = opaque(c16_);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 fa, fb[4];
          fa = frag_cols(wset[u] + (4 * ks + wt) * STRIP, 0, 0, ac2);
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) fb[kk] = frag_cols(ct, 32 * ks, 16 * (4 * team + kk), ac16);
          sched_ds_reads<10>();
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) dbp[kk] = mfma(fa, fb[kk], dbp[kk]);
          sched_mfmas<4>();
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c0 = 16 * (4 * team + k), r0 = j0 + 16 * wt;
#pragma unroll
      for (int e = 0; e < 4; ++e) store_f32(rdb.ptr(), dbp[k][e] + dbs[k][e], gn_voff(r0, c0, e), gn_soff(r0, c0, e));
    }
    if (jb + 1 < nb) {
      lds_barrier();  // the strips in the Gamma slot and C tile jb are no longer read
      load_first_gam(jb + 1);
      // B rows of block jb into C tile jb's slot, for the dC of the later passes
      tile_async<64, 16, FW>(sCt + jb * TILE_N, rb.get(), j0 * GNb + goff, GNb, vj, nch);
    }
  }  // pass

  // ---- ddt of this workgroup's heads over its chunk, then, in the last
  // workgroup to finish, dA_log and dD (bwd_dt_kernel's work, in its order of
  // operations): ds_t from the per-row sums, da_t its reverse cumsum inside
  // the chunk, ddt_t = colE_t + R'_t + A da_t, and the chunk's dA partial
  // sum_t dt_t da_t.  The per-row sums are this workgroup's own stores; the
  // barrier's fence makes every wave's stores visible to the others.  One
  // wave per head, lane l holding rows l + 64 e; eight heads at a time, their
  // ddt staged in the B tile's slot so that the stores run along the heads.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  float* const sT = reinterpret_cast<float*>(sB_);  // [QMAX][FW]
  static_assert(QMAX * FW * 4 <= TILE_N, "ddt staging fits the B tile's slot");
  const int tid = threadIdx.x;
  const int hfirst = g * hpg + sp * hps;  // the workgroup's heads hfirst .. hfirst + hps - 1
  for (int hh0 = 0; hh0 < hps; hh0 += FW) {
    const int hn = min(FW, hps - hh0);
    if (w < hn) {
      const int h = hfirst + hh0 + w;
      const int64_t o0 = sum0 + static_cast<int64_t>(h) * T;
      const float A = -__expf(A_log[h]);
      float cE[4], rP[4], rM[4], dE[4], dS[4], dv[4], ds[4];
      float sl = 0.f, tr = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = 64 * e + l;
        cE[e] = rP[e] = rM[e] = dE[e] = dS[e] = dv[e] = 0.f;
        if (k < Q) {
          // through the descriptors the passes stored with (their bases stay
          // in registers anyway): element (h, k) at byte (h T + k) 4
          const uint32_t vk = static_cast<uint32_t>(k) * 4, sh = static_cast<uint32_t>(h) * T * 4;
          cE[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rcol.ptr(), vk, sh, 0));
          rP[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rrp.ptr(), vk, sh, 0));
          dE[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rdiag.ptr(), vk, sh, 0));
          dS[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rdso.ptr(), vk, sh, 0));
          for (int jb = 0; jb <= (k >> 6); ++jb) rM[e] += s.rowM[jb * bht + o0 + k];
          dv[e] = bf16_bits_to_f32(dt[(row0 + k) * H + h]);
        }
        ds[e] = rM[e] - dv[e] * (cE[e] - dE[e]) + dS[e] - dv[e] * rP[e];
        sl += dv[e] * A;
        tr += dv[e] * rP[e];
      }
      const float ghl = l < FUSED_GH_SLOTS ? s.gh_part[((static_cast<int64_t>(bi) * nc + c) * H + h) * FUSED_GH_SLOTS + l] : 0.f;
      sl = wave_tot(sl);  // s at the chunk's last row
      tr = wave_tot(tr);
      const float gh = wave_tot(ghl);
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
        carry += lane_last(sc);
      }
      float pa = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = 64 * e + l;
        const float da = carry - incl[e] + ds[e];
        if (k < Q) sT[k * FW + w] = cE[e] + rP[e] + A * da;
        pa += dv[e] * da;
      }
      pa = wave_tot(pa);
      if (l == 0)
        __hip_atomic_store(s.dA_part + (static_cast<int64_t>(bi) * nc + c) * H + h, pa, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    for (int i = tid; i < Q * hn; i += FT) {
      const int k = i / hn, j = i - k * hn;
      ddt[(row0 + k) * H + hfirst + hh0 + j] = sT[k * FW + j];
    }
    __syncthreads();
  }
  // every wave's partial stores are complete before the workgroup counts itself
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __shared__ int sFinal;
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(s.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sFinal = prev + 1 == gridDim.x;
  }
  __syncthreads();
  if (!sFinal) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  // the last workgroup: thread tid adds head h0 + tid % hb over the chunks
  // tid / hb, tid / hb + np, ...; then one thread per head adds the np slices
  float* const sFin = reinterpret_cast<float*>(sG_);  // [2][FT]
  static_assert(2 * FT * 4 <= FW * STRIP, "final sums fit the strips' slot");
  const int64_t nbc = batch * nc;
  for (int h0 = 0; h0 < H; h0 += FT) {
    const int hb = min(FT, H - h0), np = FT / hb;
    const int hh = tid % hb, part = tid / hb;
    float a = 0.f, dd = 0.f;
    if (part < np) {
      for (int64_t v = part; v < nbc; v += np) {
        a += __hip_atomic_load(s.dA_part + v * H + h0 + hh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int ib = 0; ib < nb; ++ib)
          dd += __hip_atomic_load(s.dD_part + (v * nb + ib) * H + h0 + hh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    sFin[tid] = a;
    sFin[FT + tid] = dd;
    __syncthreads();
    if (tid < hb) {
      float ta = 0.f, td = 0.f;
      for (int p = 0; p < np; ++p) {
        ta += sFin[p * hb + tid];
        td += sFin[FT + p * hb + tid];
      }
      dA_log_out[h0 + tid] = -__expf(A_log[h0 + tid]) * ta;
      dD_out[h0 + tid] = td;
    }
    __syncthreads();
  }
  // the next call counts from 0 again
  if (tid == 0) __hip_atomic_store(s.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_bwd_fused_bf16(const Dims& d, int nsplit, const void* x, const void* B, const void* C,
                                 const void* dt, const void* dy, const float* A_log, const float* D,
                                 const void* gamma, const void* hbf, float* dx, float* dB_out, float* dC_out,
                                 float* ddt, float* dA_log, float* dD, const BwdScratch& s, hipStream_t st) {
  const int64_t nblk = static_cast<int64_t>(d.b) * d.nc() * d.G * nsplit;
  const bool full = d.P == PMAX && d.N == NMAX && d.Q == QMAX;
  hipLaunchKernelGGL(full ? bwd_fused_bf16_kernel<true> : bwd_fused_bf16_kernel<false>, dim3(static_cast<unsigned>(nblk)),
                     dim3(FT), 0, st,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(B), static_cast<const uint16_t*>(C),
                     static_cast<const uint16_t*>(dt), static_cast<const uint16_t*>(dy), A_log, D,
                     static_cast<const uint16_t*>(gamma), static_cast<const uint16_t*>(hbf), dx, dB_out, dC_out, ddt,
                     dA_log, dD, s, d.T, d.H, d.P, d.N, d.G, d.Q, nsplit);
  return hipGetLastError();
}

}  // namespace ssd
