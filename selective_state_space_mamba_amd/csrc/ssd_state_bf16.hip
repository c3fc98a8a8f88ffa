// Inter-chunk state passing (forward) and the reverse-time state-gradient pass
// (backward) for bf16 operands, with asynchronous LDS staging (ssd_async.hpp).
// Same recurrences and outputs as chunk_state_kernel (ssd_state.hip):
//
//   H_{c+1}   = exp(s_end) H_c + sum_j exp(s_end - s_j) dt_j x_j (outer) B_j
//   Gamma_c   = exp(s_end) Gamma_{c+1} + sum_i exp(s_i) dy_i (outer) C_i
//   (Gamma_nc = the gradient of the final state, zero unless given)
//
// (reference page, burn_dragon_kernel src/sequence/mamba2/backward.rs: the recurrence of
// ssd_forward_state_history_reference and the carry of ssd_backward_reference,
// unrolled over one chunk).
//
// A workgroup owns 32 headdim rows of one (batch, head); wave w holds rows
// p0 + 16 (w % 2) .. +15 and d_state columns 32 (w / 2) .. +31 of the state
// in registers and walks the chunks in order (or in reverse).  The MFMAs
// produce the state transposed (d_state along the accumulator rows), so a
// lane holds four consecutive d_state columns of one headdim row; at a chunk
// end the wave passes its part through LDS (the buffer of the chunk's last
// slab) and stores it in whole 128-byte rows, 16 bytes a lane (the state
// stores were the kernel's largest cost as 4-byte and 2-byte stores).  Per chunk the
// weighted sum is one MFMA contraction over time: the x (or dy) tile arrives
// with time along its rows, is scaled in place by the per-step weights (one
// 16-byte chunk per thread, once for the four waves that read each row) and
// is read down its rows with the LDS transpose read; the B (or C) tile
// likewise, unscaled.  Tiles come in slabs of 128 steps (64 when the grid
// is larger than one workgroup per CU, so that two share a CU),
// double-buffered and copied asynchronously while the previous slab
// computes, together with the chunk's dt series and (backward, when H_c is
// read) the f32 state tile H_c.  Every wave
// computes the within-chunk scan itself (DPP) into its own weight row.
#include "ssd_async.hpp"
#include "ssd_common.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {
constexpr int SW = 8;              // waves per workgroup
constexpr int ST = SW * WAVE;      // threads
constexpr int SPB = 32;            // headdim rows per workgroup
constexpr int HTILE = SPB * 512;   // bytes of a 32 x 128 f32 state tile
constexpr int SROW = 36;           // floats per staged state row

// Sum over all 64 lanes of the wave (the row sums end in lanes 15, 31, 47, 63).
__device__ __forceinline__ float wave_total(float v) {
  const int b = __builtin_bit_cast(int, row_sum16(v));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 15)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 31)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 47)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 63));
}
}  // namespace

// SSJ: time steps per slab (128; 64 for grids of several rounds, whose LDS
// then lets two workgroups share a CU).  HAS_H: the reverse pass reads H_c
// (for the <Gamma_{c+1}, H_c> partials or its bf16 copy).
// Kernels with 64-step slabs are held to 80 VGPRs, the budget of three
// workgroups (six waves a SIMD) on one CU.
template <bool REV, int SSJ, bool HAS_H>
__global__ __launch_bounds__(ST) __attribute__((amdgpu_waves_per_eu(SSJ == 64 ? 6 : 1))) void chunk_state_bf16_kernel(
    const uint16_t* __restrict__ X,     // fwd: x; bwd: dy       [b,T,H,P]
    const uint16_t* __restrict__ Bm,    // fwd: B; bwd: C        [b,T,G,N]
    const uint16_t* __restrict__ dt,    // [b,T,H]
    const float* __restrict__ A_log,    // [H]
    const float* __restrict__ init,     // fwd: initial state; bwd: Gamma_nc, the final state's gradient (nullable)
    float* __restrict__ states_f32,     // fwd: H_c [b,nc,H,P,N]
    uint16_t* __restrict__ states_bf,   // fwd: H_c in bf16 (nullable); bwd: Gamma_{c+1} in bf16
    float* __restrict__ last_out,       // fwd: final state; bwd: d(initial state) (nullable)
    const float* __restrict__ hstates,  // bwd: H_c (read only when gh_part or hbf_out is given)
    float* __restrict__ gh_part,        // bwd: [b,nc,H,ceil(P/16)] partial <Gamma_{c+1}, H_c> (nullable)
    uint16_t* __restrict__ hbf_out,     // bwd: H_c in bf16 (nullable)
    unsigned* __restrict__ counter,     // bwd: an arrival counter of the next kernel, zeroed here (nullable)
    int T, int H, int P, int N, int G, int Q) {
  constexpr int XSLAB = SSJ * 64;   // bytes of an SSJ x 32 bf16 slab
  constexpr int BSLAB = SSJ * 256;  // bytes of an SSJ x 128 bf16 slab
  constexpr int SLAB = BSLAB + XSLAB;  // one buffer: the B (C) slab, then the x (dy) slab
  static_assert(!HAS_H || REV, "H_c is read by the reverse pass only");
  __shared__ __attribute__((aligned(1024))) char sS_[2 * SLAB];
  __shared__ __attribute__((aligned(1024))) char sH_[HAS_H ? 2 * HTILE : 16];  // bwd: H_c (f32), two chunks
  __shared__ __attribute__((aligned(16))) float sWt[SW][QMAX];                // per-wave step weights
  __shared__ __attribute__((aligned(16))) uint32_t sDtb[2][QMAX];             // dt bits of a chunk, two chunks
  __shared__ float sGh[2][SW];
  // At a chunk end each wave stages its 16 x 32 part of the state, row-major
  // with rows padded to 36 floats (the 16 rows of a 16-byte write fall in
  // distinct banks), in the slab buffer the chunk's last slab used, to store
  // it in whole 128-byte rows.  Without an area of its own the kernel takes
  // 51 KB of LDS, so three workgroups share a CU.
  static_assert(SW * 16 * SROW * 4 <= SLAB, "the staging areas fit in one slab buffer");
  lds_char* const sS = lds_ptr(sS_);
  lds_char* const sH = lds_ptr(sH_);

  if (REV && counter && blockIdx.x == 0 && threadIdx.x == 0)
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int npb = (P + SPB - 1) / SPB, npb16 = (P + 15) / 16;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int pb = lb % npb, h = (lb / npb) % H, bi = lb / (npb * H);
  const int p0 = pb * SPB;
  const int g = h / (H / G);
  const int nc = T / Q;
  const int nsl = (Q + SSJ - 1) / SSJ;
  const float A = -__expf(A_log[h]);
  const int l = lane_id(), w = wave_id(), r = l & 15, q = l >> 4;
  const int pw = w & 1, nw = w >> 1;
  const ColsAt<4> c4_ = cols_at<4>();    // per-lane fragment offsets of the x (dy) and
  const ColsAt<16> c16_ = cols_at<16>();  // B (C) slabs
  const int64_t HP = static_cast<int64_t>(H) * P, GN = static_cast<int64_t>(G) * N;
  const int64_t PN = static_cast<int64_t>(P) * N;
  const uint32_t HPb = static_cast<uint32_t>(HP) * 2, GNb = static_cast<uint32_t>(GN) * 2;
  const int pch = min(4, (P - p0) >> 3), nch = N >> 3;
  constexpr bool need_h = HAS_H;
  float* const wts = sWt[w];

  f4 st[2];  // row p = p0 + 16 pw + r, columns n = 32 nw + 16 t + 4q + e
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p = p0 + 16 * pw + r, n = 32 * nw + 16 * t + 4 * q + e;
      st[t][e] = (init && p < P && n < N) ? init[(static_cast<int64_t>(bi) * H + h) * PN + p * N + n] : 0.f;
    }

  auto chunk_of = [&](int it) { return REV ? nc - 1 - it : it; };
  // slab copies: one descriptor per chunk (a descriptor spans 2 GiB and its
  // offsets are 32-bit, so a base per batch row would stop reaching the data
  // once a row holds 2 GiB of x), the slab's first row as the scalar offset,
  // the per-lane offsets computed once
  TileLanes<SSJ, 4, SW> lx;
  TileLanes<SSJ, 16, SW> lbs;
  lx.init(HPb, pch);
  lbs.init(GNb, nch);
  // slab sl of chunk it; with the first slab also the chunk's dt (to LDS, so
  // that no load the compiler can see is in flight: its own wait for one would
  // be vmcnt(0) and hold up every copy) and (bwd) H_c
  auto load_slab = [&](int it, int sl) {
    const int c = chunk_of(it);
    const int64_t crow = static_cast<int64_t>(bi) * T + static_cast<int64_t>(c) * Q;  // the chunk's first row
    const i32x4 rsX = make_rsrc(X + crow * HP);
    const i32x4 rsB = make_rsrc(Bm + crow * GN);
    const uint32_t t0 = static_cast<uint32_t>(sl * SSJ);  // the slab's first step in the chunk
    const int vr = min(SSJ, Q - sl * SSJ);
    const int buf = (it * nsl + sl) & 1;
    lx.issue(sS + buf * SLAB + BSLAB, rsX, t0 * HPb + static_cast<uint32_t>(h * P + p0) * 2, vr);
    lbs.issue(sS + buf * SLAB, rsB, t0 * GNb + static_cast<uint32_t>(g * N) * 2, vr);
    if (sl == 0) {
      steps_async<SW>(lds_ptr(sDtb[it & 1]), make_rsrc(dt + (static_cast<int64_t>(bi) * T + static_cast<int64_t>(c) * Q) * H + h),
                      H * 2, Q);
      if (need_h) {
        const int64_t sbase = ((static_cast<int64_t>(bi) * nc + c) * H + h) * PN + static_cast<int64_t>(p0) * N;
        tile_async<SPB, 32, SW>(sH + (it & 1) * HTILE, make_rsrc(hstates + sbase), 0, N * 4, P - p0, N >> 2);
      }
    }
  };

  load_slab(0, 0);
  for (int it = 0; it < nc; ++it) {
    const int c = chunk_of(it);
    f4 acc[2];
    zero(acc);
    float s_end = 0.f;
    for (int sl = 0; sl < nsl; ++sl) {
      wait_vm<0>();
      __syncthreads();  // slab (it, sl) visible; the other buffer is free
      if (sl == 0) {
        // this chunk's step weights (every wave computes the scan itself)
        float d[4], a[4];
        const uint4 db = *reinterpret_cast<const uint4*>(&sDtb[it & 1][4 * l]);
        const uint32_t dbv[4] = {db.x, db.y, db.z, db.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = bf16_bits_to_f32(static_cast<uint16_t>(dbv[e]));
        a[0] = d[0] * A;
#pragma unroll
        for (int e = 1; e < 4; ++e) a[e] = a[e - 1] + d[e] * A;
        const float incl = wave_scan(a[3]);
        const float ex = incl - a[3];
        const int last = Q - 1;
        s_end = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex + a[last & 3]), last >> 2));
        float wv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float s = ex + a[e];
          wv[e] = (4 * l + e < Q) ? (REV ? __expf(s) : __expf(s_end - s) * d[e]) : 0.f;
        }
        *reinterpret_cast<float4*>(wts + 4 * l) = make_float4(wv[0], wv[1], wv[2], wv[3]);
      }
      const int buf = (it * nsl + sl) & 1;
      // the slab's x rows times their step weights, in place: one 16-byte
      // chunk per thread (the swizzle keeps chunks inside their row; with
      // 64-step slabs half the threads), so that the four waves sharing a row
      // do not each scale it
      static_assert(XSLAB <= ST * 16, "at most one chunk of the x slab per thread");
      if (XSLAB == ST * 16 || static_cast<int>(threadIdx.x) < XSLAB / 16) {
        uint4* const cp = reinterpret_cast<uint4*>(sS_ + buf * SLAB + BSLAB) + threadIdx.x;
        const float wt = wts[sl * SSJ + (threadIdx.x >> 2)];
        const uint4 v = *cp;
        const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          o[k] = pack_bf16(__uint_as_float(vv[k] << 16) * wt, __uint_as_float(vv[k] & 0xFFFF0000u) * wt);
        *cp = make_uint4(o[0], o[1], o[2], o[3]);
      }
      // the next slab (or the next chunk's first, with its dt) starts loading
      if (sl + 1 < nsl)
        load_slab(it, sl + 1);
      else if (it + 1 < nc)
        load_slab(it + 1, 0);
      lds_barrier();  // the scaled slab is visible
      const lds_char* xs = sS + buf * SLAB + BSLAB;
      const lds_char* bs = sS + buf * SLAB;
      const int kw = min(SSJ, Q - sl * SSJ);
      if (kw == SSJ) {
        // a full slab: every fragment read first, then the MFMAs, so that the
        // reads' latencies overlap
        constexpr int KS = SSJ / 32;
        const ColsAt<4> ac4 = opaque(c4_);
        const ColsAt<16> ac16 = opaque(c16_);
        bf16x8 xa[KS], bb[KS][2];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          xa[ks] = frag_cols(xs, 32 * ks, 16 * pw, ac4);
#pragma unroll
          for (int t = 0; t < 2; ++t) bb[ks][t] = frag_cols(bs, 32 * ks, 32 * nw + 16 * t, ac16);
        }
        sched_ds_reads<KS * 6>();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int t = 0; t < 2; ++t) acc[t] = mfma(bb[ks][t], xa[ks], acc[t]);
      } else {
        for (int k0 = 0; k0 < kw; k0 += 32) {
          const bf16x8 ax = frag_cols<4>(xs, k0, 16 * pw);
#pragma unroll
          for (int t = 0; t < 2; ++t) acc[t] = mfma(frag_cols<16>(bs, k0, 32 * nw + 16 * t), ax, acc[t]);
        }
      }
    }

    // chunk end
    const float decay = __expf(s_end);
    const int64_t sbase = ((static_cast<int64_t>(bi) * nc + c) * H + h) * PN;
    const float* ht = reinterpret_cast<const float*>(sH_ + (it & 1) * HTILE);
    float gh = 0.f;
    // elements (p, n0 ..) of the chunk's state at byte (p N + n0) * size (N
    // is a multiple of 8, so a lane's 4 or 8 are valid together); invalid
    // ones get an out-of-range offset and their stores are dropped
    const __amdgpu_buffer_rsrc_t rsf = make_rsrc_opt(!REV && states_f32 ? states_f32 + sbase : nullptr);
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc_opt(states_bf ? states_bf + sbase : nullptr);
    const __amdgpu_buffer_rsrc_t rhb = make_rsrc_opt(hbf_out ? hbf_out + sbase : nullptr);
    // the wave's part (rows 16 pw + i, columns 32 nw + j) to its staging
    // area, once every wave is done with the last slab's buffer (the next
    // copy into it is issued after the next barrier); the same wave reads it
    // back (LDS accesses of a wave are in order)
    lds_barrier();
    float* const stg = reinterpret_cast<float*>(sS_ + ((it * nsl + nsl - 1) & 1) * SLAB) + w * 16 * SROW;
#pragma unroll
    for (int t = 0; t < 2; ++t)
      *reinterpret_cast<float4*>(stg + r * SROW + 16 * t + 4 * q) = make_float4(st[t][0], st[t][1], st[t][2], st[t][3]);
    if (!REV && states_f32) {
      // f32: rows i = l / 8 (+ 8), four columns j = 4 (l % 8) a lane
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = (l >> 3) + 8 * u, j = 4 * (l & 7), p = p0 + 16 * pw + i, n0 = 32 * nw + j;
        const float4 v = *reinterpret_cast<const float4*>(stg + i * SROW + j);
        const f4 vv = {v.x, v.y, v.z, v.w};
        store_f32x4(rsf, vv, p < P && n0 < N ? static_cast<uint32_t>(p * N + n0) * 4 : OOB_OFFSET, 0);
      }
    }
    {
      // bf16: row i = l / 4, eight columns j = 8 (l % 4) a lane
      const int i = l >> 2, j = 8 * (l & 3), p = p0 + 16 * pw + i, n0 = 32 * nw + j;
      const bool ok = p < P && n0 < N;
      const uint32_t eo = ok ? static_cast<uint32_t>(p * N + n0) * 2 : OOB_OFFSET;
      const float4 a = *reinterpret_cast<const float4*>(stg + i * SROW + j);
      const float4 b = *reinterpret_cast<const float4*>(stg + i * SROW + j + 4);
      if constexpr (!REV) {
        if (states_bf) store_bf16x8(rsb, a, b, eo, 0);
      } else {
        // H_c at the same elements (tile rows are 128 floats)
        float4 ha = make_float4(0.f, 0.f, 0.f, 0.f), hb = ha;
        if (ok && need_h) {
          ha = *reinterpret_cast<const float4*>(ht + (16 * pw + i) * NMAX + n0);
          hb = *reinterpret_cast<const float4*>(ht + (16 * pw + i) * NMAX + n0 + 4);
        }
        store_bf16x8(rsb, a, b, eo, 0);
        gh += a.x * ha.x + a.y * ha.y + a.z * ha.z + a.w * ha.w + b.x * hb.x + b.y * hb.y + b.z * hb.z + b.w * hb.w;
        if (hbf_out) store_bf16x8(rhb, ha, hb, eo, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) st[t][e] = decay * st[t][e] + acc[t][e];
    if (REV && gh_part) {
      // per 16-row headdim block (waves with the same pw), summed after the next barrier
      gh = wave_total(gh);
      if (l == 0) sGh[it & 1][w] = gh;
      if (it > 0 && threadIdx.x < 2) {
        const int cp = chunk_of(it - 1), pbi = 2 * pb + threadIdx.x;
        const float* v = sGh[(it - 1) & 1];
        if (pbi < npb16)
          gh_part[((static_cast<int64_t>(bi) * nc + cp) * H + h) * npb16 + pbi] =
              v[threadIdx.x] + v[threadIdx.x + 2] + v[threadIdx.x + 4] + v[threadIdx.x + 6];
      }
    }
  }
  if (REV && gh_part) {
    __syncthreads();
    if (threadIdx.x < 2) {
      const int cp = chunk_of(nc - 1), pbi = 2 * pb + threadIdx.x;
      const float* v = sGh[(nc - 1) & 1];
      if (pbi < npb16)
        gh_part[((static_cast<int64_t>(bi) * nc + cp) * H + h) * npb16 + pbi] =
            v[threadIdx.x] + v[threadIdx.x + 2] + v[threadIdx.x + 4] + v[threadIdx.x + 6];
    }
  }
  if (last_out) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int p = p0 + 16 * pw + r, n0 = 32 * nw + 16 * t + 4 * q;
      if (p < P && n0 < N)
        *reinterpret_cast<float4*>(last_out + (static_cast<int64_t>(bi) * H + h) * PN + p * N + n0) =
            make_float4(st[t][0], st[t][1], st[t][2], st[t][3]);
    }
  }
}

namespace {
// Compute units of the current device (looked up once).
int device_cus() {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 256;
    return n > 0 ? n : 256;
  }();
  return cus;
}
}  // namespace

// Grids of more workgroups than CUs take 64-step slabs: 51 KB of LDS, so
// three workgroups share a CU (block slice: 768 workgroups in one round); a
// grid of one round keeps 128-step slabs, with half the barriers per chunk
// (grouped workload: 36 us against 43 with 64 steps).
// The reverse pass that reads H_c (two 16 KB f32 tiles more) keeps 128.
hipError_t launch_chunk_state_fwd_bf16(const Dims& d, const void* x, const void* B, const void* dt,
                                       const float* A_log, const float* init, float* states, float* final_state,
                                       void* hbf, hipStream_t st) {
  const int64_t nblk = static_cast<int64_t>(d.b) * d.H * ((d.P + SPB - 1) / SPB);
  auto kern = nblk > device_cus() ? chunk_state_bf16_kernel<false, 64, false> : chunk_state_bf16_kernel<false, 128, false>;
  hipLaunchKernelGGL(kern, dim3(nblk), dim3(ST), 0, st, static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(B), static_cast<const uint16_t*>(dt), A_log, init, states,
                     static_cast<uint16_t*>(hbf), final_state, nullptr, nullptr, nullptr, nullptr, d.T, d.H, d.P, d.N,
                     d.G, d.Q);
  return hipGetLastError();
}

hipError_t launch_chunk_state_bwd_bf16(const Dims& d, const void* dy, const void* C, const void* dt,
                                       const float* A_log, const float* dfinal, const float* states, void* gamma,
                                       float* dinit, float* gh_part, void* hbf, unsigned* counter, hipStream_t st) {
  const int64_t nblk = static_cast<int64_t>(d.b) * d.H * ((d.P + SPB - 1) / SPB);
  const bool has_h = gh_part != nullptr || hbf != nullptr;
  auto kern = has_h ? chunk_state_bf16_kernel<true, 128, true>
                    : nblk > device_cus() ? chunk_state_bf16_kernel<true, 64, false>
                                          : chunk_state_bf16_kernel<true, 128, false>;
  hipLaunchKernelGGL(kern, dim3(nblk), dim3(ST), 0, st, static_cast<const uint16_t*>(dy),
                     static_cast<const uint16_t*>(C), static_cast<const uint16_t*>(dt), A_log, dfinal, nullptr,
                     static_cast<uint16_t*>(gamma), dinit, states, gh_part, static_cast<uint16_t*>(hbf), counter, d.T,
                     d.H, d.P, d.N, d.G, d.Q);
  return hipGetLastError();
}

}  // namespace ssd
