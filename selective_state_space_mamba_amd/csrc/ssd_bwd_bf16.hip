// Intra-chunk backward of the SSD for bf16 operands, with asynchronous LDS
// staging (ssd_async.hpp).  Same outputs and formulas as the column and row
// kernels of ssd_chunk_bwd.hip (derived there from the reverse-time loop of the
// reference page, burn_dragon_kernel src/sequence/mamba2/backward.rs,
// ssd_backward_reference), organised so that each wave's chain of
// contractions stays inside the wave.
//
// Column kernel: a workgroup owns the 64 columns j of block jb of one chunk
// for the heads of one group (or a run of them), and then those of block
// nb - 1 - jb.  Its 8 waves form two teams; wave (team, wt) owns columns
// j0 + 16 wt .. +15 and, in every 64-row block ib >= jb, the rows
// i0 + 32 team .. +31.  C.B^T for those tiles is formed once (MFMA) and kept
// in registers, as are the wave's x fragments for the head.  One step handles
// one head and one block ib; in it the wave
//   * forms yx^T = x_j . dy_i for its 16 x 32 tile with MFMA,
//   * applies the decay: G = L CB (to a wave-private LDS strip, bf16),
//     E = G yx (column and diagonal sums) and W = L yx dt_j (summed over heads
//     in registers),
//   * after a barrier, accumulates dx_j += sum_i G_ij dy_i for half of the
//     headdim columns over all 64 rows of the block (its own strip and its
//     partner wave's), reading G and dy down their rows with the LDS transpose
//     read.
// After the blocks of a head the teams add their column-sum halves through
// LDS and the state terms B_j Gamma^T and x_j Gamma follow.  At the end,
// dB_j = sum_i W_ij C_i + state terms, each team finishing half of the
// d_state columns.  The other workgroup barrier ends a step, where the next
// step's tiles (loaded by all waves while this step computed) become visible.
// The copies are issued from inline assembly, so the compiler adds no waits
// of its own for them; the kernels wait with counted vmcnt waits and use
// barriers that wait for LDS operations only.
//
// Off the diagonal block every i exceeds every j, so with s non-increasing
// L_ij = exp(s_i - s_i0) exp(s_i0 - s_j) (i0 the block's first row): factors
// <= 1 per row and per column instead of one exponential per element.
#include "ssd_async.hpp"
#include "ssd_common.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {
constexpr int BW = 8;               // waves per workgroup
constexpr int BT = BW * WAVE;       // threads per workgroup
constexpr int TILE_N = 64 * 256;    // bytes of a 64 x 128 bf16 tile
constexpr int TILE_P = 64 * 128;    // bytes of a 64 x 64 bf16 tile
constexpr int STRIP = 32 * 32;      // bytes of a 32 x 16 bf16 strip
// k-steps of 32 over the largest headdim and d_state: tiles are zero past the
// problem's P and N, so the contractions always run over the full tiles
constexpr int KP = PMAX / 32;
constexpr int KN = NMAX / 32;
static_assert(NBMAX <= 4, "the dB and dC phases hold at most four blocks' W strips");
}  // namespace

__global__ __launch_bounds__(BT) void bwd_col_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm,
    const uint16_t* __restrict__ dt, const uint16_t* __restrict__ dy, const float* __restrict__ A_log,
    const float* __restrict__ D, const uint16_t* __restrict__ gamma, float* __restrict__ dx,
    float* __restrict__ dB_out, float* __restrict__ colE, float* __restrict__ diagE, float* __restrict__ Rp,
    int T, int H, int P, int N, int G, int Q, int nsplit) {
  __shared__ __attribute__((aligned(1024))) char sB_[TILE_N];          // B rows j of block jb
  __shared__ __attribute__((aligned(1024))) char sX_[2 * TILE_P];      // x rows j, two heads; C tile slot
  __shared__ __attribute__((aligned(1024))) char sDy0_[TILE_P];        // dy rows i, even steps
  __shared__ __attribute__((aligned(1024))) char sDy1_[TILE_P];        // dy rows i, odd steps
  __shared__ __attribute__((aligned(1024))) char sGam_[TILE_N];        // Gamma [p][n]; C tile slot
  __shared__ __attribute__((aligned(1024))) char sG_[BW * STRIP];      // per-wave strips [i][j]
  __shared__ __attribute__((aligned(1024))) char sCt_[NBMAX * TILE_N];  // C tiles of blocks ib, tile ib at ib * 16 KB
  __shared__ float sRed[2][BQ][3];                                     // column sums, diagonal, R' halves
  __shared__ __attribute__((aligned(16))) float sS[2][QMAX];
  __shared__ __attribute__((aligned(16))) float sDt[2][QMAX];
  __shared__ __attribute__((aligned(16))) uint32_t sDtb[QMAX];  // dt bits of the next head to scan
  lds_char* const sB = lds_ptr(sB_);
  lds_char* const sX = lds_ptr(sX_);
  lds_char* const sDy[2] = {lds_ptr(sDy0_), lds_ptr(sDy1_)};
  lds_char* const sGam = lds_ptr(sGam_);
  lds_char* const sG = lds_ptr(sG_);
  lds_char* const sCt = lds_ptr(sCt_);

  const int nc = T / Q, nb = (Q + BQ - 1) / BQ;
  const int hpg = H / G, hps = hpg / nsplit;
  // blocks k and nb - 1 - k share a workgroup, one after the other, so that
  // every workgroup has the same number of (row block, column block) pairs
  const int npair = (nb + 1) >> 1;
  int idx = xcd_logical_block(blockIdx.x, gridDim.x);
  const int kpair = idx % npair;
  idx /= npair;
  const int sp = idx % nsplit;
  idx /= nsplit;
  const int g = idx % G;
  idx /= G;
  const int c = idx % nc;
  const int bi = idx / nc;

  for (int pass = 0; pass < 2; ++pass) {
  const int jb = pass ? nb - 1 - kpair : kpair;  // the block with the most rows i first
  if (pass && jb == kpair) break;
  if (pass) __syncthreads();

  const int l = lane_id(), w = wave_id(), r = l & 15, q = l >> 4;
  const int team = w >> 2, wt = w & 3;
  const int ti = 32 * team;  // this team's rows inside every 64-row block
  // per-lane fragment offsets (tiles of 2, 8 and 16 chunks per row)
  const RowsAt<8> r8_ = rows_at<8>();
  const RowsAt<16> r16_ = rows_at<16>();
  const ColsAt<2> c2_ = cols_at<2>();
  const ColsAt<8> c8_ = cols_at<8>();
  const ColsAt<16> c16_ = cols_at<16>();
  const AccAt<8> a8_ = acc_at<8>();
  const int64_t row0 = static_cast<int64_t>(bi) * T + static_cast<int64_t>(c) * Q;
  const int j0 = jb * BQ, vj = min(BQ, Q - j0);
  const int nib = nb - jb;
  const int64_t HP = static_cast<int64_t>(H) * P, GN = static_cast<int64_t>(G) * N;
  const uint32_t HPb = static_cast<uint32_t>(HP) * 2, GNb = static_cast<uint32_t>(GN) * 2;
  const uint32_t goff = static_cast<uint32_t>(g) * N * 2;
  const int pch = P >> 3, nch = N >> 3;
  const i32x4 rx = make_rsrc(x + row0 * HP);
  const i32x4 rdy = make_rsrc(dy + row0 * HP);
  const i32x4 rb = make_rsrc(Bm + row0 * GN);
  const i32x4 rc = make_rsrc(Cm + row0 * GN);
  const i32x4 rg = make_rsrc(gamma + (static_cast<int64_t>(bi) * nc + c) * HP * N);
  // outputs: dx from the chunk's first row; the per-column sums of (bi, h = 0, c)
  const __amdgpu_buffer_rsrc_t rdx = make_rsrc_ptr(dx + row0 * HP);
  const int64_t sum0 = static_cast<int64_t>(bi) * H * T + static_cast<int64_t>(c) * Q;
  const __amdgpu_buffer_rsrc_t rcol = make_rsrc_ptr(colE + sum0);
  const __amdgpu_buffer_rsrc_t rdiag = make_rsrc_ptr(diagE + sum0);
  const __amdgpu_buffer_rsrc_t rrp = make_rsrc_ptr(Rp + sum0);
  // the second block of a pair takes the heads in reverse order, so that the
  // heads' tiles the first block read last are still in L2
  auto headp = [&](int pp, int hh) { return g * hpg + sp * hps + (pp ? hps - 1 - hh : hh); };
  auto head = [&](int hh) { return headp(pass, hh); };

  // the dt series of head h to LDS (one copy instruction per wave; no load
  // the compiler can see, whose wait would be vmcnt(0) and hold up the copies)
  auto load_dt_abs = [&](int h) { steps_async<BW>(lds_ptr(sDtb), make_rsrc(dt + row0 * H + h), H * 2, Q); };
  auto load_dt = [&](int hh) { load_dt_abs(head(hh)); };
  // x and dy tiles (64 rows of headdim) and Gamma (headdim rows of d_state):
  // per-lane offsets computed once, the tile's first row as the scalar offset
  TileLanes<64, 8, BW> tl8;
  TileLanes<64, 16, BW> tlg;
  tl8.init(HPb, pch);
  tlg.init(N * 2, nch);
  auto load_x = [&](int hh) { tl8.issue(sX + (hh & 1) * TILE_P, rx, j0 * HPb + head(hh) * P * 2, vj); };
  auto load_dy = [&](int hh, int u, lds_char* dst) {
    const int i0 = (jb + u) * BQ;
    tl8.issue(dst, rdy, i0 * HPb + head(hh) * P * 2, min(BQ, Q - i0));
  };
  auto load_gam_abs = [&](int h) { tlg.issue(sGam, rg, h * P * N * 2, P); };
  auto load_gam = [&](int hh) { load_gam_abs(head(hh)); };
  // B rows, the first head's x, dy, Gamma and dt for column block jx of pass
  // pp (this pass, or the next while this one finishes)
  auto load_first = [&](int jx, int pp) {
    const int jx0 = jx * BQ, vjx = min(BQ, Q - jx0), h0 = headp(pp, 0);
    tile_async<64, 16, BW>(sB, rb, jx0 * GNb + goff, GNb, vjx, nch);
    tl8.issue(sX, rx, jx0 * HPb + h0 * P * 2, vjx);
    tl8.issue(sDy[0], rdy, jx0 * HPb + h0 * P * 2, vjx);
    load_gam_abs(h0);
    load_dt_abs(h0);
  };
  // the C tiles of blocks ib >= jb, each to its own 16 KB
  auto load_cs = [&]() {
#pragma unroll
    for (int u = 0; u < NBMAX; ++u) {
      if (u < nib) {
        const int i0 = (jb + u) * BQ;
        tile_async<64, 16, BW>(sCt + (jb + u) * TILE_N, rc, i0 * GNb + goff, GNb, min(BQ, Q - i0), nch);
      }
    }
  };

  // ---- B rows of block jb, the C tiles of blocks ib >= jb and the first
  // head's tiles, in flight together, then C.B^T for every block ib >= jb.
  // The C tiles stay for the dB phase and for the second block of a pair
  // (whose blocks are a subset); its first tiles load during the first
  // block's dB phase.
  if (pass == 0) {
    load_first(jb, pass);
    load_cs();
  }
  wait_vm<0>();
  __syncthreads();
  // C.B^T stays in registers for the whole block: tiles (rows j of this wave,
  // columns i = (jb + u) * 64 + ti + 16 tt + r)
  // This wave's B rows j, the first operand of C.B^T and of every head's
  // B_j Gamma^T, also stay in registers.
  f4 cbk[NBMAX][2];
  bf16x8 bfr[KN];
  {
    const RowsAt<16> ar16 = opaque(r16_);
#pragma unroll
    for (int ks = 0; ks < KN; ++ks) bfr[ks] = frag_rows(sB, 16 * wt, 4 * ks, ar16);
  }
#pragma unroll
  for (int u = 0; u < NBMAX; ++u) {
    zero(cbk[u]);
    if (u < nib) {
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
  scan_store(sDtb, -__expf(A_log[head(0)]), sS[0], sDt[0]);
  __syncthreads();

  f4 ws[NBMAX][2];  // sum over heads of L yx dt: rows j, columns i as in cbk
  f4 dbs[4];        // state part of dB: rows j, columns n = 16 (4 team + k) + r
#pragma unroll
  for (int u = 0; u < NBMAX; ++u) zero(ws[u]);
  zero(dbs);

  for (int hh = 0; hh < hps; ++hh) {
    const int h = head(hh), hb = hh & 1;
    const lds_char* xt = sX + hb * TILE_P;
    const float* sSh = sS[hb];
    const float* sDh = sDt[hb];
    float sj[4], dtj[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int jq = j0 + 16 * wt + 4 * q + e;
      sj[e] = sSh[min(jq, Q - 1)];
      dtj[e] = (jq < Q) ? sDh[jq] : 0.f;
    }
    f4 dxa[2];  // sum over rows i of G_ij dy_i: rows j, columns p = 16 (2 team + k) + r
    zero(dxa);
    float Dh = 0.f, An = 0.f;  // D of this head, A_log of the next (read at its first step)
    // column factors exp(s_i0 - s_j) <= 1 of the current off-diagonal block
    // (i0 its first row), formed at the first such block and then carried:
    // each further block multiplies them by exp(s_i0 - s_i0'), the factor of
    // the block advance (s does not increase, so every factor is <= 1)
    float cfc[4], sprev = 0.f;
    float csum[4] = {0.f, 0.f, 0.f, 0.f}, dsum[4] = {0.f, 0.f, 0.f, 0.f};
    u32x2 dsk[2];  // dy_j at columns p = ti + 16 k + r, accumulator layout
    // this wave's x rows j, the first operand of every step's yx, read once
    bf16x8 xf[KP];
    {
      const RowsAt<8> ar8 = opaque(r8_);
#pragma unroll
      for (int ks = 0; ks < KP; ++ks) xf[ks] = frag_rows(xt, 16 * wt, 4 * ks, ar8);
    }

#pragma unroll
    for (int u = 0; u < NBMAX; ++u) {
      if (u < nib) {
        const RowsAt<8> ar8 = opaque(r8_);
        const ColsAt<2> ac2 = opaque(c2_);
        const ColsAt<8> ac8 = opaque(c8_);
        const int i0 = (jb + u) * BQ;
        const lds_char* dyt = sDy[u & 1];
        // the next block's dy tile starts loading now; at a head's first step
        // the next head's dt, issued last so that the step's end need not
        // wait for it (this head's Gamma was loaded during the previous
        // head's state step)
        if (u + 1 < nib) load_dy(hh, u + 1, sDy[(u + 1) & 1]);
        if (u == 0) {
          Dh = D[h];
          if (hh + 1 < hps) {
            An = A_log[head(hh + 1)];
            load_dt(hh + 1);
          }
        }

        // yx^T: rows j (this wave's 16), columns i = i0 + ti + 16 tt + r; the
        // C.B^T tiles and the s values of the step are read with the fragments
        f4 yx[2];
        zero(yx);
        f4 cbt[2];
        float sv[2];  // s at rows i = i0 + ti + 16 tt + r (clamped)
        float sref;   // s at the block's first row
        // this lane's first row i, taken as computed here, so that the clamps
        // and masks below are made in the step (not hoisted out of the head
        // loop into spilled registers)
        const int ib0 = opaque_index(i0 + ti + r);
        {
          bf16x8 fb[KP][2];
#pragma unroll
          for (int ks = 0; ks < KP; ++ks)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) fb[ks][tt] = frag_rows(dyt, ti + 16 * tt, 4 * ks, ar8);
          cbt[0] = cbk[u][0];
          cbt[1] = cbk[u][1];
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) sv[tt] = sSh[min(ib0 + 16 * tt, Q - 1)];
          sref = sSh[i0];
          sched_ds_reads<2 * KP + 3>();
#pragma unroll
          for (int ks = 0; ks < KP; ++ks)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) yx[tt] = mfma(xf[ks], fb[ks][tt], yx[tt]);
          sched_mfmas<2 * KP>();
        }
        f4 gv[2];
        if (u == 0) {
          const int jq0 = opaque_index(j0 + 16 * wt + 4 * q);
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int iq = ib0 + 16 * tt;
            const float si = sv[tt];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int jq = jq0 + e;
              const float ex = __expf(si - sj[e]);
              const float L = (iq < Q && iq >= jq) ? ex : 0.f;
              const float G1 = L * cbt[tt][e];
              const float E = G1 * yx[tt][e];
              csum[e] += E;
              if (iq == jq) dsum[e] += E;
              ws[u][tt][e] += L * dtj[e] * yx[tt][e];
              gv[tt][e] = G1;
            }
          }
          const AccAt<8> aa8 = opaque(a8_);
#pragma unroll
          for (int k = 0; k < 2; ++k) dsk[k] = block_acc(dyt, 16 * wt, ti + 16 * k, aa8);
        } else {
          float cf[4], cfd[4];
          if (u == 1) {
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
            const float rx = __expf(sv[tt] - sref);
            const float rf = (iq < Q) ? rx : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float G1 = rf * cf[e] * cbt[tt][e];
              const float E = G1 * yx[tt][e];
              csum[e] += E;
              ws[u][tt][e] += rf * cfd[e] * yx[tt][e];
              gv[tt][e] = G1;
            }
          }
        }
        put_strip(sG + w * STRIP, gv);
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
        if (u == 0 && hh + 1 < hps)
          wait_vm<1>();  // all but the dt copy
        else
          wait_vm<0>();
        lds_barrier();
      }
    }

    // ---- state terms of head hh; the next head's x and dy tiles start
    // loading, its Gamma once this head's is read
    const RowsAt<16> ar16 = opaque(r16_);
    const ColsAt<16> ac16 = opaque(c16_);
    if (hh + 1 < hps) {
      load_x(hh + 1);
      load_dy(hh + 1, 0, sDy[0]);
    }
    f4 bg[2];  // B_j Gamma^T: rows j, columns p = 16 (2 team + k) + r
    zero(bg);
#pragma unroll
    for (int kh = 0; kh < KN; kh += 2) {  // two k-steps per batch of reads
      bf16x8 fb[2][2];
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int k = 0; k < 2; ++k) fb[d][k] = frag_rows(sGam, 16 * (2 * team + k), 4 * (kh + d), ar16);
      sched_ds_reads<4>();
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int k = 0; k < 2; ++k) bg[k] = mfma(bfr[kh + d], fb[d][k], bg[k]);
      sched_mfmas<4>();
    }
    // x_j Gamma for this team's d_state columns (the state part of dB)
    f4 v[4];
    zero(v);
#pragma unroll
    for (int ks = 0; ks < KP; ++ks) {
      bf16x8 fb[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) fb[k] = frag_cols(sGam, 32 * ks, 16 * (4 * team + k), ac16);
      sched_ds_reads<8>();
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = mfma(xf[ks], fb[k], v[k]);
      sched_mfmas<4>();
    }
    u32x2 xa[2];  // x_j at columns p = 16 (2 team + k) + r, accumulator layout
    {
      const AccAt<8> aa8 = opaque(a8_);
#pragma unroll
      for (int k = 0; k < 2; ++k) xa[k] = block_acc(xt, 16 * wt, 16 * (2 * team + k), aa8);
    }
    const float s_end = sSh[Q - 1];
    float wj[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int jl = 16 * wt + 4 * q + e;
      const float wx = __expf(s_end - sj[e]);
      wj[e] = (j0 + jl < Q) ? wx : 0.f;
      float part = 0.f;
#pragma unroll
      for (int k = 0; k < 2; ++k) part += bg[k][e] * acc_elem(xa[k], e);
      part = row_sum16(part);
      const float cs = row_sum16(csum[e]), ds = row_sum16(dsum[e]);
      if (r == 15) {
        sRed[team][jl][0] = cs;
        sRed[team][jl][1] = ds;
        sRed[team][jl][2] = wj[e] * part;
      }
    }
    if (hh + 1 < hps) wait_vm<2>();  // the next head's dt copy (its x and dy copies may be in flight)
    lds_barrier();
    if (hh + 1 < hps) load_gam(hh + 1);  // this head's Gamma is no longer read
    float dxv[2][4];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) dxv[k][e] = dtj[e] * (dxa[k][e] + wj[e] * bg[k][e]) + Dh * acc_elem(dsk[k], e);
    // the per-column sums of this wave's columns j = 16 wt + (l % 16), one
    // column per lane of each 16-lane row
    const int jc = 16 * wt + r;
    const float ce = sRed[0][jc][0] + sRed[1][jc][0];
    const float de = sRed[0][jc][1] + sRed[1][jc][1];
    const float re = sRed[0][jc][2] + sRed[1][jc][2];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float f = dtj[e] * wj[e];
#pragma unroll
      for (int k = 0; k < 4; ++k) dbs[k][e] += f * v[k][e];
    }
    // the next head's x and dy tiles (all but Gamma's 2 copies) must be in
    // LDS at the barrier; the stores below are issued after the wait and
    // complete during the next step
    if (hh + 1 < hps) wait_vm<2>();
    // dx (element (jq, p) at byte (jq HP + h P + p) 4 from the chunk's first
    // row) and the per-column sums; out-of-range offsets are dropped
    {
      const uint32_t vdx = (static_cast<uint32_t>(j0 + 16 * wt + 4 * q) * HP + 32 * team + r) * 4;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = j0 + 16 * wt + 4 * q + e < Q && 32 * team + 16 * k + r < P;
          store_f32(rdx, dxv[k][e], ok ? vdx + 64 * k : OOB_OFFSET, static_cast<uint32_t>(e * HP + h * P) * 4);
        }
      }
      if (team == 0) {
        const uint32_t vo = (q == 0 && j0 + jc < Q) ? static_cast<uint32_t>(j0 + jc) * 4 : OOB_OFFSET;
        const uint32_t so = static_cast<uint32_t>(h) * T * 4;
        store_f32(rcol, ce, vo, so);
        store_f32(rdiag, de, vo, so);
        store_f32(rrp, re, vo, so);
      }
    }
    if (hh + 1 < hps) scan_store(sDtb, -__expf(An), sS[hb ^ 1], sDt[hb ^ 1]);
    lds_barrier();
  }

  // ---- dB_j = sum_i W_ij C_i + state terms, for this team's d_state columns
  // over all rows i (own and partner strips), against the C tiles of the
  // prologue.  The W strips of blocks u = 0..2 go
  // to wset[u] (block 3, if any, reuses wset[0] after them), leaving the B,
  // first x, first dy and Gamma tiles free for the next pass's first tiles,
  // which start loading now.
  if (pass == 0 && nb - 1 - kpair != kpair) load_first(nb - 1 - kpair, 1);
  f4 dbp[4];
  zero(dbp);
  lds_char* const wset[3] = {sG, sX + TILE_P, sDy[1]};
  auto db_block = [&](int u, const lds_char* ws_strips) {
    const lds_char* ct = sCt + (jb + u) * TILE_N;
    const ColsAt<2> ac2 = opaque(c2_);
    const ColsAt<16> ac16 = opaque(c16_);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 fa, fb[4];
      fa = frag_cols(ws_strips + (4 * ks + wt) * STRIP, 0, 0, ac2);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) fb[kk] = frag_cols(ct, 32 * ks, 16 * (4 * team + kk), ac16);
      sched_ds_reads<10>();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) dbp[kk] = mfma(fa, fb[kk], dbp[kk]);
      sched_mfmas<4>();
    }
  };
#pragma unroll
  for (int u = 0; u < 3; ++u)
    if (u < nib) put_strip(wset[u] + w * STRIP, ws[u]);
  lds_barrier();
#pragma unroll
  for (int u = 0; u < 3; ++u)
    if (u < nib) db_block(u, wset[u]);
  if (nib > 3) {
    lds_barrier();
    put_strip(wset[0] + w * STRIP, ws[3]);
    lds_barrier();
    db_block(3, wset[0]);
  }
  const int64_t batch = gridDim.x / (npair * nsplit * G * nc);
  float* dBo = dB_out + static_cast<int64_t>(sp) * batch * T * GN;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int n = 16 * (4 * team + k) + r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int jq = j0 + 16 * wt + 4 * q + e;
      if (jq < Q && n < N) dBo[(row0 + jq) * GN + static_cast<int64_t>(g) * N + n] = dbp[k][e] + dbs[k][e];
    }
  }
  }  // pass
}

// Row kernel: a workgroup owns the 64 rows i of block ib of one chunk for the
// heads of one group (or a run of them); wave (team, wt) owns rows
// i0 + 16 wt .. +15 and, in every block jb <= ib, the columns j0 + 32 team
// .. +31.  C_i.B_j for those tiles is formed once and kept in registers, as
// are the wave's dy fragments for the head.  A step
// (one head, one block jb) forms yx = dy_i . x_j with MFMA and applies the
// decay: W = L yx dt_j (summed over heads in registers) and the strictly-lower
// row sums of M = W CB.  Once per head: U_i = dy_i H_c with MFMA (H_c as bf16,
// read down its rows with the LDS transpose read), the readout term
// exp(s_i) U_i . C_i, and the head sum of exp(s_i) U_i; dD is the diagonal of
// yx.  At the end dC_i = sum_j W_ij B_j + sum_h exp(s_i) U_i, each team
// finishing half of the d_state columns.
__global__ __launch_bounds__(BT) void bwd_row_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm,
    const uint16_t* __restrict__ dt, const uint16_t* __restrict__ dy, const float* __restrict__ A_log,
    const uint16_t* __restrict__ hbf, float* __restrict__ dC_out, float* __restrict__ rowM,
    float* __restrict__ dsoff, float* __restrict__ dD_part, unsigned* __restrict__ done, int T, int H, int P,
    int N, int G, int Q, int nsplit) {
  __shared__ __attribute__((aligned(1024))) char sC_[TILE_N];          // C rows i of block ib
  __shared__ __attribute__((aligned(1024))) char sDy_[2 * TILE_P];     // dy rows i, two heads; B tile slot
  __shared__ __attribute__((aligned(1024))) char sX0_[TILE_P];         // x rows j, even steps
  __shared__ __attribute__((aligned(1024))) char sX1_[TILE_P];         // x rows j, odd steps
  __shared__ __attribute__((aligned(1024))) char sH_[TILE_N];          // H_c [p][n] (bf16); B tile slot
  __shared__ __attribute__((aligned(1024))) char sG_[BW * STRIP];      // per-wave W strips [j][i]
  __shared__ __attribute__((aligned(1024))) char sBt_[NBMAX * TILE_N];  // B tiles of blocks jb, tile jb at jb * 16 KB
  __shared__ float sRed[2][BQ][2];                                     // row-sum and readout halves
  __shared__ float sDD[BW][4];                                         // dD partials
  __shared__ __attribute__((aligned(16))) float sS[2][QMAX];
  __shared__ __attribute__((aligned(16))) float sDt[2][QMAX];
  __shared__ __attribute__((aligned(16))) uint32_t sDtb[QMAX];  // dt bits of the next head to scan
  lds_char* const sC = lds_ptr(sC_);
  lds_char* const sDy = lds_ptr(sDy_);
  lds_char* const sX[2] = {lds_ptr(sX0_), lds_ptr(sX1_)};
  lds_char* const sH = lds_ptr(sH_);
  lds_char* const sG = lds_ptr(sG_);
  lds_char* const sBt = lds_ptr(sBt_);

  const int nc = T / Q, nb = (Q + BQ - 1) / BQ;
  const int hpg = H / G, hps = hpg / nsplit;
  // blocks nb - 1 - k and k share a workgroup, one after the other
  const int npair = (nb + 1) >> 1;
  int idx = xcd_logical_block(blockIdx.x, gridDim.x);
  const int kpair = idx % npair;
  idx /= npair;
  const int sp = idx % nsplit;
  idx /= nsplit;
  const int g = idx % G;
  idx /= G;
  const int c = idx % nc;
  const int bi = idx / nc;

  for (int pass = 0; pass < 2; ++pass) {
  const int ib = pass ? kpair : nb - 1 - kpair;  // the block with the most columns j first
  if (pass && ib == nb - 1 - kpair) break;
  if (pass) __syncthreads();

  const int l = lane_id(), w = wave_id(), r = l & 15, q = l >> 4;
  const int team = w >> 2, wt = w & 3;
  const int tj = 32 * team;  // this team's columns inside every 64-column block
  // per-lane fragment offsets (tiles of 2, 8 and 16 chunks per row)
  const RowsAt<8> r8_ = rows_at<8>();
  const RowsAt<16> r16_ = rows_at<16>();
  const ColsAt<2> c2_ = cols_at<2>();
  const ColsAt<16> c16_ = cols_at<16>();
  const AccAt<16> a16_ = acc_at<16>();
  const int64_t row0 = static_cast<int64_t>(bi) * T + static_cast<int64_t>(c) * Q;
  const int i0 = ib * BQ, vi = min(BQ, Q - i0);
  const int nj = ib + 1;
  const int64_t HP = static_cast<int64_t>(H) * P, GN = static_cast<int64_t>(G) * N;
  const uint32_t HPb = static_cast<uint32_t>(HP) * 2, GNb = static_cast<uint32_t>(GN) * 2;
  const uint32_t goff = static_cast<uint32_t>(g) * N * 2;
  const int pch = P >> 3, nch = N >> 3;
  const i32x4 rx = make_rsrc(x + row0 * HP);
  const i32x4 rdy = make_rsrc(dy + row0 * HP);
  const i32x4 rb = make_rsrc(Bm + row0 * GN);
  const i32x4 rc = make_rsrc(Cm + row0 * GN);
  const i32x4 rh = make_rsrc(hbf + (static_cast<int64_t>(bi) * nc + c) * HP * N);
  // outputs: the per-row sums of (bi, h = 0, c)
  const int64_t sum0 = static_cast<int64_t>(bi) * H * T + static_cast<int64_t>(c) * Q;
  const __amdgpu_buffer_rsrc_t rrow = make_rsrc_ptr(rowM + sum0);
  const __amdgpu_buffer_rsrc_t rdso = make_rsrc_ptr(dsoff + sum0);
  // the second block of a pair takes the heads in reverse order, so that the
  // heads' tiles the first block read last are still in L2
  auto headp = [&](int pp, int hh) { return g * hpg + sp * hps + (pp ? hps - 1 - hh : hh); };
  auto head = [&](int hh) { return headp(pass, hh); };

  // the dt series of head h to LDS (one copy instruction per wave; no load
  // the compiler can see, whose wait would be vmcnt(0) and hold up the copies)
  auto load_dt_abs = [&](int h) { steps_async<BW>(lds_ptr(sDtb), make_rsrc(dt + row0 * H + h), H * 2, Q); };
  auto load_dt = [&](int hh) { load_dt_abs(head(hh)); };
  // x and dy tiles (64 rows of headdim) and H_c (headdim rows of d_state):
  // per-lane offsets computed once, the tile's first row as the scalar offset
  TileLanes<64, 8, BW> tl8;
  TileLanes<64, 16, BW> tlh;
  tl8.init(HPb, pch);
  tlh.init(N * 2, nch);
  auto load_x = [&](int hh, int jb, lds_char* dst) {
    const int j0 = jb * BQ;
    tl8.issue(dst, rx, j0 * HPb + head(hh) * P * 2, min(BQ, Q - j0));
  };
  auto load_dy = [&](int hh) { tl8.issue(sDy + (hh & 1) * TILE_P, rdy, i0 * HPb + head(hh) * P * 2, vi); };
  auto load_h_abs = [&](int h) { tlh.issue(sH, rh, h * P * N * 2, P); };
  auto load_h = [&](int hh) { load_h_abs(head(hh)); };
  // C rows, the first head's dy, first x, H_c and dt for row block ix of
  // pass pp (this pass, or the next while this one finishes)
  auto load_first = [&](int ix, int pp) {
    const int ix0 = ix * BQ, vix = min(BQ, Q - ix0), h0 = headp(pp, 0);
    tile_async<64, 16, BW>(sC, rc, ix0 * GNb + goff, GNb, vix, nch);
    tl8.issue(sDy, rdy, ix0 * HPb + h0 * P * 2, vix);
    tl8.issue(sX[0], rx, h0 * P * 2, min(BQ, Q));
    load_h_abs(h0);
    load_dt_abs(h0);
  };
  // the B tiles of blocks jb <= ib, each to its own 16 KB
  auto load_bs = [&]() {
#pragma unroll
    for (int jb = 0; jb < NBMAX; ++jb) {
      if (jb < nj) {
        const int j0 = jb * BQ;
        tile_async<64, 16, BW>(sBt + jb * TILE_N, rb, j0 * GNb + goff, GNb, min(BQ, Q - j0), nch);
      }
    }
  };

  // ---- C rows of block ib, the B tiles of blocks jb <= ib and the first
  // head's tiles, in flight together, then C.B^T for every block jb <= ib.
  // The B tiles stay for the dC phase and for the second block of a pair
  // (whose blocks are a subset); its first tiles load during the first
  // block's dC phase.
  if (pass == 0) {
    load_first(ib, pass);
    load_bs();
  }
  wait_vm<0>();
  __syncthreads();
  // C.B^T stays in registers for the whole block: tiles (rows i of this wave,
  // columns j = jb * 64 + tj + 16 tt + r)
  f4 cbk[NBMAX][2];
  bf16x8 cfr[KN];  // this wave's C rows i, read once for every block jb
  {
    const RowsAt<16> ar16 = opaque(r16_);
#pragma unroll
    for (int ks = 0; ks < KN; ++ks) cfr[ks] = frag_rows(sC, 16 * wt, 4 * ks, ar16);
  }
#pragma unroll
  for (int jb = 0; jb < NBMAX; ++jb) {
    zero(cbk[jb]);
    if (jb < nj) {
      const lds_char* bt = sBt + jb * TILE_N;
      const RowsAt<16> ar16 = opaque(r16_);
      bf16x8 fb[KN][2];
#pragma unroll
      for (int ks = 0; ks < KN; ++ks)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) fb[ks][tt] = frag_rows(bt, tj + 16 * tt, 4 * ks, ar16);
      sched_ds_reads<2 * KN>();
#pragma unroll
      for (int ks = 0; ks < KN; ++ks)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) cbk[jb][tt] = mfma(cfr[ks], fb[ks][tt], cbk[jb][tt]);
      sched_mfmas<2 * KN>();
    }
  }
  scan_store(sDtb, -__expf(A_log[head(0)]), sS[0], sDt[0]);
  __syncthreads();

  u32x2 ca[4];  // C_i at columns n = 16 (4 team + k) + r, accumulator layout, for every head
  {
    const AccAt<16> aa16 = opaque(a16_);
#pragma unroll
    for (int k = 0; k < 4; ++k) ca[k] = block_acc(sC, 16 * wt, 16 * (4 * team + k), aa16);
  }
  f4 ws[NBMAX][2];  // sum over heads of L yx dt: rows i, columns j = jb * 64 + tj + 16 tt + r
  f4 ua[4];         // sum over heads of exp(s_i) U_i: rows i, columns n = 16 (4 team + k) + r
#pragma unroll
  for (int jb = 0; jb < NBMAX; ++jb) zero(ws[jb]);
  zero(ua);

  for (int hh = 0; hh < hps; ++hh) {
    const int h = head(hh), hb = hh & 1;
    const lds_char* dyt = sDy + hb * TILE_P;
    const float* sSh = sS[hb];
    const float* sDh = sDt[hb];
    float si[4], rf[4];
    const float sref = sSh[i0];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int iq = i0 + 16 * wt + 4 * q + e;
      si[e] = sSh[min(iq, Q - 1)];
      const float ex = __expf(si[e] - sref);
      rf[e] = (iq < Q) ? ex : 0.f;
    }
    float rm[4] = {0.f, 0.f, 0.f, 0.f};  // strictly-lower row sums of M over this team's columns
    float ddv = 0.f;                     // diagonal of yx
    float An = 0.f;                      // A_log of the next head (read at this head's first step)
    // this wave's dy rows i, the first operand of every step's yx and of U
    bf16x8 dyf[KP];
    {
      const RowsAt<8> ar8 = opaque(r8_);
#pragma unroll
      for (int ks = 0; ks < KP; ++ks) dyf[ks] = frag_rows(dyt, 16 * wt, 4 * ks, ar8);
    }

#pragma unroll
    for (int jb = 0; jb < NBMAX; ++jb) {
      if (jb < nj) {
        const int j0 = jb * BQ;
        const lds_char* xt = sX[jb & 1];
        // the next block's x tile starts loading now; at a head's first step
        // the next head's dt, issued last so that the step's end need not
        // wait for it (this head's H_c was loaded during the previous head's
        // per-head terms)
        if (jb + 1 < nj) load_x(hh, jb + 1, sX[(jb + 1) & 1]);
        if (jb == 0 && hh + 1 < hps) {
          An = A_log[head(hh + 1)];
          load_dt(hh + 1);
        }
        // yx: rows i (this wave's 16), columns j = j0 + tj + 16 tt + r; the
        // C.B^T tiles and the s and dt values of the columns are read with the
        // fragments
        const RowsAt<8> ar8 = opaque(r8_);
        f4 yx[2];
        zero(yx);
        f4 cbt[2];
        float sjv[2], dtv[2];  // s and dt at columns j = j0 + tj + 16 tt + r (clamped)
        // this lane's first column j, taken as computed here (clamps and masks
        // made in the step, not hoisted into spilled registers)
        const int jb0 = opaque_index(j0 + tj + r);
        {
          bf16x8 fb[KP][2];
#pragma unroll
          for (int ks = 0; ks < KP; ++ks)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) fb[ks][tt] = frag_rows(xt, tj + 16 * tt, 4 * ks, ar8);
          cbt[0] = cbk[jb][0];
          cbt[1] = cbk[jb][1];
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int jc = min(jb0 + 16 * tt, Q - 1);
            sjv[tt] = sSh[jc];
            dtv[tt] = sDh[jc];
          }
          sched_ds_reads<2 * KP + 4>();
#pragma unroll
          for (int ks = 0; ks < KP; ++ks)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) yx[tt] = mfma(dyf[ks], fb[ks][tt], yx[tt]);
          sched_mfmas<2 * KP>();
        }
        if (jb == ib) {
          const int iq0 = opaque_index(i0 + 16 * wt + 4 * q);
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int jq = jb0 + 16 * tt;
            const float sj = sjv[tt];
            const float dtj = (jq < Q) ? dtv[tt] : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int iq = iq0 + e;
              const float ex = __expf(si[e] - sj);
              const float L = (iq < Q && jq <= iq) ? ex : 0.f;
              const float ly = L * yx[tt][e] * dtj;
              ws[jb][tt][e] += ly;
              if (jq < iq) rm[e] += ly * cbt[tt][e];
              if (jq == iq) ddv += yx[tt][e];
            }
          }
        } else {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const float cfd = __expf(sref - sjv[tt]) * dtv[tt];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float ly = rf[e] * cfd * yx[tt][e];
              ws[jb][tt][e] += ly;
              rm[e] += ly * cbt[tt][e];
            }
          }
        }
        if (jb == 0 && hh + 1 < hps)
          wait_vm<1>();  // all but the dt copy
        else
          wait_vm<0>();
        lds_barrier();
      }
    }

    // ---- per-head terms; the next head's dy and x tiles start loading, its
    // H_c once this head's is read
    if (hh + 1 < hps) {
      load_dy(hh + 1);
      load_x(hh + 1, 0, sX[0]);
    }
    f4 u[4];  // U_i = dy_i H_c: rows i, columns n = 16 (4 team + k) + r
    zero(u);
    {
      const RowsAt<8> ar8 = opaque(r8_);
      const ColsAt<16> ac16 = opaque(c16_);
#pragma unroll
      for (int ks = 0; ks < KP; ++ks) {
        bf16x8 fb[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) fb[k] = frag_cols(sH, 32 * ks, 16 * (4 * team + k), ac16);
        sched_ds_reads<8>();
#pragma unroll
        for (int k = 0; k < 4; ++k) u[k] = mfma(dyf[ks], fb[k], u[k]);
        sched_mfmas<4>();
      }
    }
    float ex[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int il = 16 * wt + 4 * q + e;
      const float xe = __expf(si[e]);
      ex[e] = (i0 + il < Q) ? xe : 0.f;
      float part = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        part += u[k][e] * acc_elem(ca[k], e);
        ua[k][e] += ex[e] * u[k][e];
      }
      part = row_sum16(part);
      const float rs = row_sum16(rm[e]);
      if (r == 15) {
        sRed[team][il][0] = rs;
        sRed[team][il][1] = ex[e] * part;
      }
    }
    {
      const float dd = row_sum16(ddv);
      if (r == 15) sDD[w][q] = dd;
    }
    if (hh + 1 < hps) wait_vm<2>();  // the next head's dt copy (its dy and x copies may be in flight)
    lds_barrier();
    if (hh + 1 < hps) load_h(hh + 1);  // this head's H_c is no longer read
    // the per-row sums of this wave's rows i = 16 wt + (l % 16), one row per
    // lane of each 16-lane row
    const int ic = 16 * wt + r;
    const float rmv = sRed[0][ic][0] + sRed[1][ic][0];
    const float dso = sRed[0][ic][1] + sRed[1][ic][1];
    float tot = 0.f;
#pragma unroll
    for (int kk = 0; kk < BW; ++kk) tot += sDD[kk][0] + sDD[kk][1] + sDD[kk][2] + sDD[kk][3];
    // the next head's dy and x tiles (all but H_c's 2 copies) must be in LDS
    // at the barrier; the stores below are issued after the wait and complete
    // during the next step
    if (hh + 1 < hps) wait_vm<2>();
    if (team == 0) {
      // out-of-range offsets are dropped
      const uint32_t vo = (q == 0 && i0 + ic < Q) ? static_cast<uint32_t>(i0 + ic) * 4 : OOB_OFFSET;
      const uint32_t so = static_cast<uint32_t>(h) * T * 4;
      store_f32(rrow, rmv, vo, so);
      store_f32(rdso, dso, vo, so);
    }
    if (threadIdx.x == 0) dD_part[((static_cast<int64_t>(bi) * nc + c) * nb + ib) * H + h] = tot;
    if (hh + 1 < hps) scan_store(sDtb, -__expf(An), sS[hb ^ 1], sDt[hb ^ 1]);
    lds_barrier();
  }

  // ---- dC_i = sum_j W_ij B_j + sum_h exp(s_i) U_i for this team's d_state
  // columns over all columns j (own and partner strips), against the B tiles
  // of the prologue.  The W strips of blocks
  // jb = 0..2 go to wset[jb] (block 3, if any, reuses wset[0] after them),
  // leaving the C, first dy, first x and H_c tiles free for the next pass's
  // first tiles, which start loading now.
  if (pass == 0 && nb - 1 - kpair != kpair) load_first(kpair, 1);
  lds_char* const wset[3] = {sG, sX[1], sDy + TILE_P};
  auto dc_block = [&](int jb, const lds_char* w_strips) {
    const lds_char* bt = sBt + jb * TILE_N;
    const ColsAt<2> ac2 = opaque(c2_);
    const ColsAt<16> ac16 = opaque(c16_);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 fa, fb[4];
      fa = frag_cols(w_strips + (4 * ks + wt) * STRIP, 0, 0, ac2);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) fb[kk] = frag_cols(bt, 32 * ks, 16 * (4 * team + kk), ac16);
      sched_ds_reads<10>();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) ua[kk] = mfma(fa, fb[kk], ua[kk]);
      sched_mfmas<4>();
    }
  };
#pragma unroll
  for (int jb = 0; jb < 3; ++jb)
    if (jb < nj) put_strip(wset[jb] + w * STRIP, ws[jb]);
  lds_barrier();
#pragma unroll
  for (int jb = 0; jb < 3; ++jb)
    if (jb < nj) dc_block(jb, wset[jb]);
  if (nj > 3) {
    lds_barrier();
    put_strip(wset[0] + w * STRIP, ws[3]);
    lds_barrier();
    dc_block(3, wset[0]);
  }
  const int64_t batch = gridDim.x / (npair * nsplit * G * nc);
  float* dCo = dC_out + static_cast<int64_t>(sp) * batch * T * GN;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int n = 16 * (4 * team + k) + r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int iq = i0 + 16 * wt + 4 * q + e;
      if (iq < Q && n < N) dCo[(row0 + iq) * GN + static_cast<int64_t>(g) * N + n] = ua[k][e];
    }
  }
  }  // pass
  // the dt kernel that follows counts its finished workgroups from 0
  if (blockIdx.x == 0 && threadIdx.x == 0) __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

bool bwd_bf16_supported(const Dims& d) {
  // Every buffer descriptor of the bf16 family starts at a chunk (x, dy, y,
  // dx, B, C, dt), at one (batch, chunk) state block (Gamma, the bf16 states)
  // or at one (batch, chunk) of the [b, H, T] per-head sums, and takes 32-bit
  // byte offsets within its 2 GiB range.  The largest offsets are a chunk of
  // f32 dx (Q H P 4), a state block (H P N 2) and a head's row of the sums
  // (H T 4); problems past these bounds take the general kernels.
  const int64_t lim = (int64_t(1) << 31) - 4096;
  const int64_t HP = int64_t(d.H) * d.P, GN = int64_t(d.G) * d.N;
  return d.P % 8 == 0 && d.N % 8 == 0 && int64_t(QMAX) * HP * 4 < lim && int64_t(QMAX) * GN * 4 < lim &&
         HP * d.N * 2 < lim && int64_t(d.H) * d.T * 4 < lim && int64_t(QMAX) * d.H * 2 < lim;
}

hipError_t launch_bwd_row_bf16(const Dims& d, int nsplit, const void* x, const void* B, const void* C,
                               const void* dt, const void* dy, const float* A_log, const void* hbf,
                               float* dC_out, const BwdScratch& s, hipStream_t st) {
  const int64_t nblk = static_cast<int64_t>(d.b) * d.nc() * d.G * nsplit * ((d.nb() + 1) / 2);
  hipLaunchKernelGGL(bwd_row_bf16_kernel, dim3(nblk), dim3(BT), 0, st, static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(B), static_cast<const uint16_t*>(C),
                     static_cast<const uint16_t*>(dt), static_cast<const uint16_t*>(dy), A_log,
                     static_cast<const uint16_t*>(hbf), dC_out, s.rowM, s.dsoff, s.dD_part, s.done, d.T, d.H, d.P, d.N,
                     d.G, d.Q, nsplit);
  return hipGetLastError();
}

hipError_t launch_bwd_col_bf16(const Dims& d, int nsplit, const void* x, const void* B, const void* C,
                               const void* dt, const void* dy, const float* A_log, const float* D,
                               const void* gamma, float* dx, float* dB_out, const BwdScratch& s,
                               hipStream_t st) {
  const int64_t nblk = static_cast<int64_t>(d.b) * d.nc() * d.G * nsplit * ((d.nb() + 1) / 2);
  hipLaunchKernelGGL(bwd_col_bf16_kernel, dim3(nblk), dim3(BT), 0, st, static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(B), static_cast<const uint16_t*>(C),
                     static_cast<const uint16_t*>(dt), static_cast<const uint16_t*>(dy), A_log, D,
                     static_cast<const uint16_t*>(gamma), dx, dB_out, s.colE, s.diagE, s.Rp, d.T, d.H, d.P,
                     d.N, d.G, d.Q, nsplit);
  return hipGetLastError();
}

}  // namespace ssd
