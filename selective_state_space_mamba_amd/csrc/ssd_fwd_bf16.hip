// Chunk output of the SSD forward for bf16 operands, with asynchronous LDS
// staging (ssd_async.hpp).  Same result as chunk_out_fwd_kernel
// (ssd_chunk_fwd.hip): for the state H_c entering chunk c and s the
// within-chunk cumsum of dt A (the recurrence of the reference page,
// burn_dragon_kernel src/sequence/mamba2/backward.rs, ssd_forward_state_history_reference,
// with the y readout of the block backward),
//
//   y_i = sum_{j<=i} exp(s_i - s_j) (C_i . B_j) dt_j x_j + exp(s_i) C_i . H_c^T + D x_i.
//
// A workgroup owns the 64 rows i of block ib of one chunk for the heads of one
// group (or a run of them), and then those of block nb - 1 - ib.  Its 8 waves
// form two teams; wave (team, wt) owns rows i0 + 16 wt .. +15 and, in every
// block jb <= ib, the columns j0 + 32 team .. +31.  C_i.B_j for those tiles is
// formed once (MFMA) and kept in registers.  A step (one head, one block jb) applies the decay and dt_j,
// puts the bf16 result in a wave-private LDS strip and accumulates
// sum_j G_ij x_j over the wave's 32 columns j with MFMA (G and x read down
// their rows with the LDS transpose read).  Once per head the teams swap the
// halves of their sums through LDS; each team finishes half of the headdim
// columns with the incoming-state term (C_i against H_c in bf16) and the skip
// term.  Workgroup barriers end steps, where the next step's tiles (loaded
// by all waves while this step computed) become visible.
//
// Off the diagonal block every j is below every i, so with s non-increasing
// L_ij = exp(s_i - s_i0) exp(s_i0 - s_j) (i0 the block's first row): factors
// <= 1 per row and per column instead of one exponential per element.
#include "ssd_async.hpp"
#include "ssd_common.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {
constexpr int FW = 8;               // waves per workgroup
constexpr int FT = FW * WAVE;       // threads per workgroup
constexpr int FTILE_N = 64 * 256;   // bytes of a 64 x 128 bf16 tile
constexpr int FTILE_P = 64 * 128;   // bytes of a 64 x 64 bf16 tile
constexpr int FSTRIP = 32 * 32;     // bytes of a 32 x 16 bf16 strip
// k-steps of 32 over the largest d_state: tiles are zero past the problem's N,
// so the contractions always run over the full tiles
constexpr int FKN = NMAX / 32;

// s and dt for t < Q from the dt bits copied to LDS, one dword per step (see
// the backward kernels).
__device__ __forceinline__ void fwd_scan_store(const uint32_t* dtb_lds, float A, float* s_out, float* dt_out) {
  const int l = lane_id(), w = wave_id();
  float d[4], a[4];
  const uint4 db = *reinterpret_cast<const uint4*>(dtb_lds + 4 * l);
  const uint32_t dbv[4] = {db.x, db.y, db.z, db.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) d[e] = bf16_bits_to_f32(static_cast<uint16_t>(dbv[e]));
  a[0] = d[0] * A;
#pragma unroll
  for (int e = 1; e < 4; ++e) a[e] = a[e - 1] + d[e] * A;
  const float incl = wave_scan(a[3]);
  const float ex = incl - a[3];
  if ((l >> 4) == w) {
    *reinterpret_cast<float4*>(s_out + 4 * l) = make_float4(ex + a[0], ex + a[1], ex + a[2], ex + a[3]);
    *reinterpret_cast<float4*>(dt_out + 4 * l) = make_float4(d[0], d[1], d[2], d[3]);
  }
}

// bf16 per staged y row: 32 columns and 8 of padding (the 16-byte rows of
// four lanes' writes fall in distinct banks; 80 bytes keeps rows 16-byte aligned)
constexpr int YROW = 40;

// Two MFMA tiles (lane element e at row 4q + e, column 16 tt + r) into a wave
// strip as bf16 [column][row] (32 x 16).
__device__ __forceinline__ void fwd_put_strip(lds_char* strip, const f4 (&v)[2]) {
  const int l = lane_id(), r = l & 15, q = l >> 4;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
    *(__attribute__((address_space(3))) u32x2*)(strip + strip_off(16 * tt + r, 8 * q)) =
        u32x2{pack_bf16(v[tt][0], v[tt][1]), pack_bf16(v[tt][2], v[tt][3])};
}
}  // namespace

__global__ __launch_bounds__(FT) __attribute__((amdgpu_waves_per_eu(4, 4))) void out_fwd_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm,
    const uint16_t* __restrict__ dt, const float* __restrict__ A_log, const float* __restrict__ D,
    const uint16_t* __restrict__ hbf, uint16_t* __restrict__ y, int T, int H, int P, int N, int G, int Q,
    int nsplit) {
  // 77 KB, so that two workgroups share a CU:
  //   C rows i of block ib (read for C.B^T and every head's C_i . H_c^T) | H_c
  //   [p][n] | x rows j of even and odd steps | per-wave G strips [j][i] | the
  //   teams' y halves | s and dt of two heads | the next head's dt bits.
  // The B tiles are needed only for C.B^T at a block's start: they pass two
  // at a time through [x odd | G strips] and [y halves] (16 KB each), which
  // are idle then.
  __shared__ __attribute__((aligned(1024))) char smem[3 * FTILE_N + 3 * FTILE_P + 5 * QMAX * 4];
  static_assert(FW * FSTRIP == FTILE_P, "the strips and the odd x tile form one 16 KB B slot");
  lds_char* const sC = lds_ptr(smem);
  lds_char* const sH = sC + FTILE_N;
  lds_char* const sX[2] = {sH + FTILE_N, sH + FTILE_N + FTILE_P};
  lds_char* const sG = sX[1] + FTILE_P;
  lds_char* const sXch = sG + FW * FSTRIP;
  lds_char* const sBslot[2] = {sXch, sX[1]};
  char* const tail = smem + 3 * FTILE_N + 3 * FTILE_P;
  float (*const sS)[QMAX] = reinterpret_cast<float (*)[QMAX]>(tail);
  float (*const sDt)[QMAX] = reinterpret_cast<float (*)[QMAX]>(tail + 2 * QMAX * 4);
  uint32_t* const sDtb = reinterpret_cast<uint32_t*>(tail + 4 * QMAX * 4);

  const int nc = T / Q, nb = (Q + BQ - 1) / BQ;
  const int hpg = H / G, hps = hpg / nsplit;
  // blocks nb - 1 - k and k share a workgroup, one after the other, so that
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
  const int ib = pass ? kpair : nb - 1 - kpair;  // the block with the most columns j first
  if (pass && ib == nb - 1 - kpair) break;
  if (pass) __syncthreads();

  const int l = lane_id(), w = wave_id(), r = l & 15, q = l >> 4;
  const int team = w >> 2, wt = w & 3;
  const int tj = 32 * team;
  // per-lane fragment offsets (tiles of 2, 8 and 16 chunks per row)
  const RowsAt<16> r16_ = rows_at<16>();
  const ColsAt<2> c2_ = cols_at<2>();
  const ColsAt<8> c8_ = cols_at<8>();
  const AccAt<8> a8_ = acc_at<8>();
  const int64_t row0 = static_cast<int64_t>(bi) * T + static_cast<int64_t>(c) * Q;
  const int i0 = ib * BQ, vi = min(BQ, Q - i0);
  const int nj = ib + 1;
  const int64_t HP = static_cast<int64_t>(H) * P, GN = static_cast<int64_t>(G) * N;
  const uint32_t HPb = static_cast<uint32_t>(HP) * 2, GNb = static_cast<uint32_t>(GN) * 2;
  const uint32_t goff = static_cast<uint32_t>(g) * N * 2;
  const int pch = P >> 3, nch = N >> 3;
  const LazyRsrc rx{x + row0 * HP};
  const LazyRsrc rb{Bm + row0 * GN};
  const LazyRsrc rc{Cm + row0 * GN};
  const LazyRsrc rh{hbf + (static_cast<int64_t>(bi) * nc + c) * HP * N};
  const LazyRsrc ry{y + row0 * HP};
  auto head = [&](int hh) { return g * hpg + sp * hps + hh; };

  // the dt series of head hh to LDS (one copy instruction per wave; no load
  // the compiler can see, whose wait would be vmcnt(0) and hold up the copies)
  auto load_dt = [&](int hh) { steps_async<FW>(lds_ptr(sDtb), make_rsrc(dt + row0 * H + head(hh)), H * 2, Q); };
  // x tiles (64 rows of headdim) and H_c (headdim rows of d_state), the
  // tile's first row as the scalar offset; the per-lane offsets are
  // recomputed at each copy (with four waves per SIMD they would not stay in
  // registers)
  auto load_x = [&](int hh, int jb, lds_char* dst) {
    const int j0 = jb * BQ;
    tile_issue_fresh<64, 8, FW>(dst, rx.get(), HPb, pch, j0 * HPb + head(hh) * P * 2, min(BQ, Q - j0));
  };
  auto load_h = [&](int hh) { tile_issue_fresh<64, 16, FW>(sH, rh.get(), N * 2, nch, head(hh) * P * N * 2, P); };
  // C rows, the first head's first x, H_c and dt for row block ix (this
  // pass's, or the next pass's while this one finishes)
  auto load_first = [&](int ix) {
    const int ix0 = ix * BQ, vix = min(BQ, Q - ix0);
    tile_async<64, 16, FW>(sC, rc.get(), ix0 * GNb + goff, GNb, vix, nch);
    load_x(0, 0, sX[0]);
    load_h(0);
    load_dt(0);
  };
  // the B tiles of blocks jp and jp + 1 (those <= ib) to the two B slots
  auto load_bpair = [&](int jp) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (jp + t < nj) {
        const int j0 = (jp + t) * BQ;
        tile_async<64, 16, FW>(sBslot[t], rb.get(), j0 * GNb + goff, GNb, min(BQ, Q - j0), nch);
      }
    }
  };
  // whether a second row block follows in this workgroup
  const bool next = pass == 0 && nb - 1 - kpair != kpair;

  // ---- C rows of block ib, the first two B tiles and the first head's
  // tiles, in flight together (the second block of a pair had its C, x, H_c
  // and dt copies issued during the first block's last head), then C.B^T for
  // every block jb <= ib, two B tiles at a time, kept in registers
  if (pass == 0) load_first(ib);
  load_bpair(0);
  wait_vm<0>();
  __syncthreads();
  // C.B^T stays in registers as bf16 pairs (it only scales the bf16 G tiles:
  // one more rounding of each element, and half the registers); this wave's C
  // rows i are read from the C tile again for every head's C_i . H_c^T.
  u32x2 cbk[NBMAX][2];  // rows i of this wave, columns j = jb * 64 + tj + 16 tt + r
  bf16x8 cfr[FKN];
  {
    const RowsAt<16> ar16 = opaque(r16_);
#pragma unroll
    for (int ks = 0; ks < FKN; ++ks) cfr[ks] = frag_rows(sC, 16 * wt, 4 * ks, ar16);
  }
#pragma unroll
  for (int jb = 0; jb < NBMAX; ++jb) {
    cbk[jb][0] = cbk[jb][1] = u32x2{0u, 0u};
    if ((jb & 1) == 0 && jb > 0 && jb < nj) {
      // the next two B tiles, once every wave has read the slots
      lds_barrier();
      load_bpair(jb);
      wait_vm<0>();
      lds_barrier();
    }
    if (jb < nj) {
      const lds_char* bt = sBslot[jb & 1];
      const RowsAt<16> ar16 = opaque(r16_);
      bf16x8 fb[FKN][2];
#pragma unroll
      for (int ks = 0; ks < FKN; ++ks)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) fb[ks][tt] = frag_rows(bt, tj + 16 * tt, 4 * ks, ar16);
      sched_ds_reads<2 * FKN>();
      f4 cb[2];
      zero(cb);
#pragma unroll
      for (int ks = 0; ks < FKN; ++ks)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) cb[tt] = mfma(cfr[ks], fb[ks][tt], cb[tt]);
      sched_mfmas<2 * FKN>();
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) cbk[jb][tt] = u32x2{pack_bf16(cb[tt][0], cb[tt][1]), pack_bf16(cb[tt][2], cb[tt][3])};
    }
  }
  lds_barrier();  // the B slots are free for the x, strip and y tiles
  fwd_scan_store(sDtb, -__expf(A_log[head(0)]), sS[0], sDt[0]);
  __syncthreads();

  for (int hh = 0; hh < hps; ++hh) {
    const int h = head(hh), hb = hh & 1;
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
    f4 ya[4];  // sum over this team's columns j of G_ij x_j: rows i, columns p = 16 pt + r
    zero(ya);
    float Dh = 0.f, An = 0.f;  // D of this head, A_log of the next (read at its first step)
    u32x2 xsk[2];  // x_i at columns p = 32 team + 16 k + r, accumulator layout

#pragma unroll
    for (int jb = 0; jb < NBMAX; ++jb) {
      if (jb < nj) {
        const int j0 = jb * BQ;
        const lds_char* xt = sX[jb & 1];
        // the next block's x tile starts loading now; at a head's first step
        // the next head's dt, issued last so that the step's end need not
        // wait for it (this head's H_c was loaded during the previous head's
        // last terms)
        if (jb + 1 < nj) load_x(hh, jb + 1, sX[(jb + 1) & 1]);
        if (jb == 0) {
          Dh = D[h];
          if (hh + 1 < hps) {
            An = A_log[head(hh + 1)];
            load_dt(hh + 1);
          }
        }
        // the s and dt values of the step's columns and the x fragments of the
        // G x contraction are read together
        const ColsAt<2> ac2 = opaque(c2_);
        const ColsAt<8> ac8 = opaque(c8_);
        f4 cbt[2];
        float sjv[2], dtv[2];  // s and dt at columns j = j0 + tj + 16 tt + r (clamped)
        bf16x8 fx[4];
        // this lane's first column j, taken as computed here (clamps and masks
        // made in the step, not hoisted into spilled registers)
        const int jb0 = opaque_index(j0 + tj + r);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e) cbt[tt][e] = acc_elem(cbk[jb][tt], e);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int jc = min(jb0 + 16 * tt, Q - 1);
          sjv[tt] = sSh[jc];
          dtv[tt] = sDh[jc];
        }
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) fx[pt] = frag_cols(xt, tj, 16 * pt, ac8);
        sched_ds_reads<12>();
        f4 gv[2];
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
              gv[tt][e] = L * dtj * cbt[tt][e];
            }
          }
          const AccAt<8> aa8 = opaque(a8_);
#pragma unroll
          for (int k = 0; k < 2; ++k) xsk[k] = block_acc(xt, 16 * wt, 32 * team + 16 * k, aa8);
        } else {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const float cfd = __expf(sref - sjv[tt]) * dtv[tt];
#pragma unroll
            for (int e = 0; e < 4; ++e) gv[tt][e] = rf[e] * cfd * cbt[tt][e];
          }
        }
        fwd_put_strip(sG + w * FSTRIP, gv);
        {
          const bf16x8 a = frag_cols(sG + w * FSTRIP, 0, 0, ac2);
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) ya[pt] = mfma(a, fx[pt], ya[pt]);
        }
        if (jb == 0 && hh + 1 < hps)
          wait_vm<1>();  // all but the dt copy
        else
          wait_vm<0>();
        lds_barrier();
      }
    }

    // ---- finish head hh; the next head's first x tile starts loading, its
    // H_c once this head's is read (after the last head, the next block's
    // first tiles)
    if (hh + 1 < hps) load_x(hh + 1, 0, sX[0]);
    // hand the other team's headdim columns to it
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int pt = 2 * (1 - team) + k;
      *(__attribute__((address_space(3))) f4*)(sXch + ((wt * 4 + pt) * WAVE + l) * 16) = ya[pt];
    }
    f4 yo[2];  // C_i . H_c^T: rows i, columns p = 16 (2 team + k) + r
    zero(yo);
    {
      const RowsAt<16> ar16 = opaque(r16_);
#pragma unroll
      for (int kh = 0; kh < FKN; kh += 2) {  // two k-steps per batch of reads
        bf16x8 fb[2][2], fc[2];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          fc[d] = frag_rows(sC, 16 * wt, 4 * (kh + d), ar16);
#pragma unroll
          for (int k = 0; k < 2; ++k) fb[d][k] = frag_rows(sH, 16 * (2 * team + k), 4 * (kh + d), ar16);
        }
        sched_ds_reads<6>();
#pragma unroll
        for (int d = 0; d < 2; ++d)
#pragma unroll
          for (int k = 0; k < 2; ++k) yo[k] = mfma(fc[d], fb[d][k], yo[k]);
        sched_mfmas<4>();
      }
    }
    if (hh + 1 < hps) wait_vm<1>();  // the next head's dt copy (its x copy may be in flight)
    lds_barrier();
    if (hh + 1 < hps)
      load_h(hh + 1);  // this head's H_c is no longer read
    else if (next)
      load_first(kpair);
    uint16_t yv[2][4];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int pt = 2 * team + k;
      const f4 other = *(const __attribute__((address_space(3))) f4*)(sXch + ((wt * 4 + pt) * WAVE + l) * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float xv = acc_elem(xsk[k], e);
        const float ex = __expf(si[e]);
        yv[k][e] = f32_to_bf16_bits(ya[pt][e] + other[e] + ex * yo[k][e] + Dh * xv);
      }
    }
    // the next head's first x tile (all but H_c's 2 copies) must be in LDS
    // at the barrier; the stores below are issued after the wait and complete
    // during the next step
    if (hh + 1 < hps) wait_vm<2>();
    // y (element (iq, p) at byte (iq HP + h P + p) 2 from the chunk's first
    // row) through this wave's two exchange slots, read above and untouched
    // by other waves until the next head's exchange, after the barrier
    // below: the wave's 16 rows x 32 columns row-major (rows padded to YROW
    // bf16), then 16 bytes a lane (row l / 4, columns 8 (l % 4) ..) as one
    // store (P is a multiple of 8, so a lane's eight are valid together);
    // out-of-range offsets are dropped
    {
      __attribute__((address_space(3))) uint16_t* const stg =
          reinterpret_cast<__attribute__((address_space(3))) uint16_t*>(sXch + (wt * 4 + 2 * team) * WAVE * 16);
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) stg[(4 * q + e) * YROW + 16 * k + r] = yv[k][e];
      const int iy = l >> 2, jy = 8 * (l & 3);
      const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(stg + iy * YROW + jy);
      const bool ok = i0 + 16 * wt + iy < Q && 32 * team + jy < P;
      const uint32_t vo = (static_cast<uint32_t>(i0 + 16 * wt + iy) * HP + h * P + 32 * team + jy) * 2;
      __builtin_amdgcn_raw_buffer_store_b128(v, ry.ptr(), ok ? vo : OOB_OFFSET, 0, 0);
    }
    if (hh + 1 < hps) fwd_scan_store(sDtb, -__expf(An), sS[hb ^ 1], sDt[hb ^ 1]);
    lds_barrier();
  }
  }  // pass
}

hipError_t launch_out_fwd_bf16(const Dims& d, int nsplit, const void* x, const void* B, const void* C,
                               const void* dt, const float* A_log, const float* D, const void* hbf, void* y,
                               hipStream_t st) {
  const int64_t nblk = static_cast<int64_t>(d.b) * d.nc() * d.G * nsplit * ((d.nb() + 1) / 2);
  hipLaunchKernelGGL(out_fwd_bf16_kernel, dim3(nblk), dim3(FT), 0, st, static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(B), static_cast<const uint16_t*>(C),
                     static_cast<const uint16_t*>(dt), A_log, D, static_cast<const uint16_t*>(hbf),
                     static_cast<uint16_t*>(y), d.T, d.H, d.P, d.N, d.G, d.Q, nsplit);
  return hipGetLastError();
}

}  // namespace ssd
