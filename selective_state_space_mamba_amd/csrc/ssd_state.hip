// Inter-chunk state passing (forward) and the reverse-time state-gradient pass
// (backward) of the chunked SSD.
//
// The recurrence h_t = exp(dt_t A) h_{t-1} + dt_t x_t (outer) B_t of the reference
// page (burn_dragon_kernel src/sequence/mamba2/backward.rs,
// ssd_forward_state_history_reference), unrolled over one chunk of Q steps with
// s_i = sum_{r<=i} dt_r A (within the chunk), gives
//
//   H_{c+1} = exp(s_end) H_c + sum_j exp(s_end - s_j) dt_j x_j (outer) B_j.
//
// The reverse-time loop of ssd_backward_reference carries
// G_t = dy_t (outer) C_t + exp(dt_{t+1} A) G_{t+1}; unrolled over a chunk,
//
//   Gamma_c = exp(s_end) Gamma_{c+1} + sum_i exp(s_i) dy_i (outer) C_i,
//
// with Gamma_nc the gradient of the final state (zero unless given) and
// d(initial state) = Gamma_0.
//
// With bf16 operands both are one kernel: a workgroup owns 16 headdim rows of
// one (batch, head) and walks the chunks in order (forward) or in reverse
// (backward), keeping its 16 x N slice of the state in registers.  Per chunk
// the weighted sum is one MFMA contraction over the chunk's time steps
// (K = Q), the operands staged in LDS in slabs.  Rows of the state are
// independent, so the headdim split needs no communication.
//
// With f32 operands (MFMA at a sixteenth of the bf16 rate) the walk would
// serialise the contractions of every chunk, so the work is split in two:
// chunk_sum_f32_kernel computes each chunk's weighted sum S_c (dS_c) with one
// workgroup per (batch, chunk, head) and writes it into the chunk's slot of
// the output, with the chunk's total log-decay s_end; state_scan_kernel then
// walks the chunks once per (batch, head, headdim block), combining
// H_{c+1} = exp(s_end) H_c + S_c (Gamma_c = exp(s_end) Gamma_{c+1} + dS_c) in
// place.  All decay factors are exp of
// non-positive numbers (dt > 0, A < 0).
#include <type_traits>

#include "ssd_common.hpp"
#include "ssd_launch.hpp"

namespace ssd {

// Time steps staged per slab: a whole chunk of up to 256 steps for bf16
// operands (64 KB of B), 128 for f32.
template <bool BF> struct StateSlab { static constexpr int SJ = BF ? 256 : 128; };

template <typename TX, typename TB, typename TDT, bool BF, bool REV>
__global__ __launch_bounds__(NTHREADS, 2) void chunk_state_kernel(
    const TX* __restrict__ X,          // fwd: x; bwd: dy            [b,T,H,P]
    const TB* __restrict__ Bm,         // fwd: B; bwd: C             [b,T,G,N]
    const TDT* __restrict__ dt,        // [b,T,H]
    const float* __restrict__ A_log,   // [H]
    const float* __restrict__ init,    // fwd: initial state; bwd: Gamma_nc, the final state's gradient (nullable)
    void* __restrict__ states_out_v,   // fwd: H_c (f32); bwd: Gamma_{c+1} (operand type) [b,nc,H,P,N]
    float* __restrict__ last_out,      // fwd: final state; bwd: d(initial state) (nullable)
    const float* __restrict__ hstates, // bwd: H_c, for <Gamma_{c+1}, H_c>
    float* __restrict__ gh_part,       // bwd: [b,nc,H,npb]
    uint16_t* __restrict__ hbf,        // bwd: H_c rounded to bf16 (nullable)
    int T, int H, int P, int N, int G, int Q) {
  typedef typename Op<BF>::T OT;
  // The forward writes the f32 chunk states; the backward writes Gamma in the
  // operand type of the kernels that read it (its only use is as an MFMA operand).
  typedef typename std::conditional<REV, OT, float>::type TSO;
  TSO* const states_out = static_cast<TSO*>(states_out_v);
  constexpr int PB = STATE_PB;
  constexpr int SJ = StateSlab<BF>::SJ;
  constexpr int LDX = SJ + (BF ? 8 : 4);  // [p][j] and [n][j]: time contiguous
  __shared__ __attribute__((aligned(16))) OT sX[PB * LDX];
  __shared__ __attribute__((aligned(16))) OT sB[NMAX * LDX];
  __shared__ float sS[QMAX];
  __shared__ float sW[QMAX];
  __shared__ float sTmp[8];

  // p-blocks of a head, then the heads of a group, are consecutive logical
  // blocks: they read the same B (or C) slab, so they share an XCD's L2.
  const int npb = (P + PB - 1) / PB;
  const int nc = T / Q;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int pb = lb % npb, h = (lb / npb) % H, bi = lb / (npb * H);
  const int p0 = pb * PB;
  const int g = h / (H / G);
  const int nslab = (Q + SJ - 1) / SJ;
  const float A = -__expf(A_log[h]);
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), r = l & 15, q = l >> 4;
  const int64_t HP = static_cast<int64_t>(H) * P, GN = static_cast<int64_t>(G) * N;
  const int64_t PN = static_cast<int64_t>(P) * N;

  // wave w holds state columns n = 32w .. 32w+31 (two 16-wide tiles) of rows p0..p0+15
  f4 st[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = p0 + 4 * q + i, n = 32 * w + 16 * t + r;
      st[t][i] = (init && p < P && n < N) ? init[(static_cast<int64_t>(bi) * H + h) * PN + p * N + n] : 0.f;
    }

  TransTile<TX, SJ, PB> tx;    // x (or dy) rows j, columns p0..p0+15 -> [p][j]
  TransTile<TB, SJ, NMAX> tb;  // B (or C) rows j -> [n][j]
  const int total = nc * nslab;
  auto chunk_of = [&](int step) { const int it = step / nslab; return REV ? nc - 1 - it : it; };
  auto prefetch = [&](int step, float& dtn) {
    const int c = chunk_of(step), sl = step % nslab;
    const int64_t row0 = static_cast<int64_t>(bi) * T + static_cast<int64_t>(c) * Q + sl * SJ;
    const int vr = min(SJ, Q - sl * SJ);
    tx.load(X + row0 * HP + static_cast<int64_t>(h) * P + p0, HP, vr, P - p0);
    tb.load(Bm + row0 * GN + static_cast<int64_t>(g) * N, GN, vr, N);
    if (sl == 0)
      dtn = (tid < Q) ? load_f(dt, (static_cast<int64_t>(bi) * T + static_cast<int64_t>(c) * Q + tid) * H + h) : 0.f;
  };
  float dt_next = 0.f;
  prefetch(0, dt_next);

  f4 acc[2];
  zero(acc);
  for (int step = 0; step < total; ++step) {
    const int c = chunk_of(step), sl = step % nslab;
    if (sl == 0) {
      const float dtv = dt_next;
      const float s = block_inclusive_scan(dtv * A, sTmp);
      if (tid < Q) sS[tid] = s;
      __syncthreads();
      const float s_end = sS[Q - 1];
      if (tid < Q) sW[tid] = REV ? __expf(s) : __expf(s_end - s) * dtv;
      zero(acc);
    }
    __syncthreads();  // sW visible; previous slab's MFMA reads of sX / sB done
    tx.store(sX, LDX, sW + sl * SJ);
    tb.store(sB, LDX);
    if (step + 1 < total) prefetch(step + 1, dt_next);
    __syncthreads();
    wave_gemm<BF, true, true, 2>(acc, sX, LDX, 1, sB + 32 * w * LDX, LDX, 1, round_up(min(SJ, Q - sl * SJ), Op<BF>::KS));
    if (sl != nslab - 1) continue;

    const int64_t sbase = ((static_cast<int64_t>(bi) * nc + c) * H + h) * PN;
    const float decay = __expf(sS[Q - 1]);
    float gh = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = p0 + 4 * q + i, n = 32 * w + 16 * t + r;
        if (p < P && n < N) {
          if (states_out) store_f(states_out, sbase + p * N + n, st[t][i]);
          if (!REV && hbf) hbf[sbase + p * N + n] = f32_to_bf16_bits(st[t][i]);
          if (REV) {
            const float hv = hstates[sbase + p * N + n];
            gh += st[t][i] * hv;
            if (hbf) hbf[sbase + p * N + n] = f32_to_bf16_bits(hv);
          }
        }
        st[t][i] = decay * st[t][i] + acc[t][i];
      }
    if (REV) {
      gh = wave_sum(gh);
      if (l == 0) sTmp[4 + w] = gh;
      __syncthreads();
      if (tid == 0)
        gh_part[((static_cast<int64_t>(bi) * nc + c) * H + h) * npb + pb] = sTmp[4] + sTmp[5] + sTmp[6] + sTmp[7];
    }
  }

  if (last_out) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = p0 + 4 * q + i, n = 32 * w + 16 * t + r;
        if (p < P && n < N) last_out[(static_cast<int64_t>(bi) * H + h) * PN + p * N + n] = st[t][i];
      }
  }
}

// First pass of the f32 form: one workgroup per (batch, chunk, head) forms the
// chunk's whole P x N weighted sum (forward S_c = sum_j exp(s_end - s_j) dt_j
// x_j (outer) B_j, backward dS_c = sum_i exp(s_i) dy_i (outer) C_i) over slabs
// of SUM_SJ steps, so each B (C) slab staged in LDS serves every headdim row
// of the head; wave w owns rows 16w .. 16w+15 and the workgroup's d_state
// columns: all of them, or (NSPL = 2, for grids under two workgroups per CU)
// one half, the two halves of a (batch, chunk, head) being adjacent blocks.
// The sum goes to the chunk's slot of `sums`, the chunk's total log-decay
// s_end to `send`.
constexpr int SUM_SJ = 64;
template <typename TX, typename TB, bool REV, int NSPL>
__global__ __launch_bounds__(NTHREADS, 2) void chunk_sum_f32_kernel(
    const TX* __restrict__ X,         // fwd: x; bwd: dy            [b,T,H,P]
    const TB* __restrict__ Bm,        // fwd: B; bwd: C             [b,T,G,N]
    const TB* __restrict__ dt,        // [b,T,H]
    const float* __restrict__ A_log,  // [H]
    float* __restrict__ sums,         // [b,nc,H,P,N]
    float* __restrict__ send,         // [b,nc,H]
    int T, int H, int P, int N, int G, int Q) {
  static_assert(NTHREADS / WAVE * 16 == PMAX, "one wave per 16 headdim rows");
  constexpr int LDX = SUM_SJ + 4;  // [p][j] and [n][j]: time contiguous, padded
  constexpr int NW = NMAX / NSPL;  // d_state columns per workgroup
  __shared__ __attribute__((aligned(16))) float sX[PMAX * LDX];
  __shared__ __attribute__((aligned(16))) float sB[NW * LDX];
  __shared__ float sW[QMAX];
  __shared__ float sTmp[8];
  const int nc = T / Q;
  int lb = xcd_logical_block(blockIdx.x, gridDim.x);  // heads of a chunk share an XCD
  const int n0 = (lb % NSPL) * NW;
  lb /= NSPL;
  const int h = lb % H, c = (lb / H) % nc, bi = lb / (H * nc);
  const int g = h / (H / G);
  const float A = -__expf(A_log[h]);
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), r = l & 15, q = l >> 4;
  const int64_t HP = static_cast<int64_t>(H) * P, GN = static_cast<int64_t>(G) * N;
  const int64_t PN = static_cast<int64_t>(P) * N;
  const int64_t row_c = static_cast<int64_t>(bi) * T + static_cast<int64_t>(c) * Q;

  TransTile<TX, SUM_SJ, PMAX, 4> tx;  // x (or dy) rows j -> [p][j], scaled by the step weights
  TransTile<TB, SUM_SJ, NW, 4> tb;    // B (or C) rows j, this workgroup's columns -> [n][j]
  const int nslab = (Q + SUM_SJ - 1) / SUM_SJ;
  auto load = [&](int sl) {
    const int64_t row0 = row_c + sl * SUM_SJ;
    const int vr = min(SUM_SJ, Q - sl * SUM_SJ);
    tx.load(X + row0 * HP + static_cast<int64_t>(h) * P, HP, vr, P);
    tb.load(Bm + row0 * GN + static_cast<int64_t>(g) * N + n0, GN, vr, min(NW, N - n0));
  };
  load(0);

  const float dtv = tid < Q ? load_f(dt, (row_c + tid) * H + h) : 0.f;
  const float s = block_inclusive_scan(dtv * A, sTmp);
  if (tid == Q - 1) sTmp[4] = s;
  __syncthreads();
  const float s_end = sTmp[4];
  if (tid < Q) sW[tid] = REV ? __expf(s) : __expf(s_end - s) * dtv;
  if (tid == 0 && n0 == 0) send[(static_cast<int64_t>(bi) * nc + c) * H + h] = s_end;

  f4 acc[NW / 16];
  zero(acc);
  for (int sl = 0; sl < nslab; ++sl) {
    __syncthreads();  // sW visible; the previous slab's reads of sX / sB done
    tx.store(sX, LDX, sW + sl * SUM_SJ);
    tb.store(sB, LDX);
    if (sl + 1 < nslab) load(sl + 1);
    __syncthreads();
    // one 4-byte read per k-step: the 16-byte reads cost this kernel a wave
    // per SIMD of occupancy and were slower (long workload 318 -> 353 us)
    wave_gemm<false, true, true, NW / 16, false>(acc, sX + 16 * w * LDX, LDX, 1, sB, LDX, 1,
                                           round_up(min(SUM_SJ, Q - sl * SUM_SJ), Op<false>::KS));
  }
  const int64_t base = ((static_cast<int64_t>(bi) * nc + c) * H + h) * PN;
#pragma unroll
  for (int t = 0; t < NW / 16; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = 16 * w + 4 * q + i, n = n0 + 16 * t + r;
      if (p < P && n < N) sums[base + p * N + n] = acc[t][i];
    }
}

// The chunk walk of the two-pass form.  A workgroup of 16 waves owns headdim
// rows p0 .. p0+15 of one (batch, head); thread t holds elements t and t + 1024
// of that contiguous 16 x N block.  Forward: slot c holds S_c on entry and H_c
// on exit, run = H_0 = init (or 0), run <- exp(s_end_c) run + S_c, last = H_nc.
// Backward: slot c holds dS_c on entry and Gamma_{c+1} on exit, run =
// Gamma_nc = init (the final state's gradient, or 0), run <- exp(s_end_c) run +
// dS_c, last = Gamma_0, and gh_part[b,c,h,pb] = <Gamma_{c+1}, H_c> over the
// block.  The values of the next four chunks (and, backward, their H_c) are in
// flight while a chunk's slot is written.
constexpr int SCAN_THREADS = 1024;
constexpr int SCAN_EPT = STATE_PB * NMAX / SCAN_THREADS;  // elements per thread
constexpr int SCAN_AHEAD = 4;                             // chunks loaded ahead
template <bool REV>
__global__ __launch_bounds__(SCAN_THREADS) void state_scan_kernel(float* __restrict__ states,
                                                                 const float* __restrict__ send,
                                                                 const float* __restrict__ init,
                                                                 float* __restrict__ last,
                                                                 const float* __restrict__ hstates,
                                                                 float* __restrict__ gh_part, int nc, int H, int P,
                                                                 int N) {
  __shared__ float sTmp[SCAN_THREADS / WAVE];
  const int npb = (P + STATE_PB - 1) / STATE_PB;
  const int lb = blockIdx.x;
  const int pb = lb % npb, h = (lb / npb) % H, bi = lb / (npb * H);
  const int p0 = pb * STATE_PB;
  const int nvalid = min(STATE_PB, P - p0) * N;  // contiguous elements of the block
  const int64_t PN = static_cast<int64_t>(P) * N;
  const int64_t off0 = static_cast<int64_t>(p0) * N;
  const int tid = threadIdx.x;
  float run[SCAN_EPT], buf[SCAN_AHEAD][SCAN_EPT];
  float hbuf[SCAN_AHEAD][SCAN_EPT];  // backward: H_c of the chunks in flight
#pragma unroll
  for (int k = 0; k < SCAN_EPT; ++k) {
    const int e = tid + SCAN_THREADS * k;
    run[k] = (init && e < nvalid) ? init[(static_cast<int64_t>(bi) * H + h) * PN + off0 + e] : 0.f;
  }
  auto chunk = [&](int it) { return REV ? nc - 1 - it : it; };
  auto slot = [&](int it) { return ((static_cast<int64_t>(bi) * nc + chunk(it)) * H + h) * PN + off0; };
  auto load = [&](int it, float (&v)[SCAN_EPT], float (&hv)[SCAN_EPT]) {
#pragma unroll
    for (int k = 0; k < SCAN_EPT; ++k) {
      const int e = tid + SCAN_THREADS * k;
      const bool ok = it < nc && e < nvalid;
      v[k] = ok ? states[slot(it) + e] : 0.f;
      if (REV) hv[k] = ok ? hstates[slot(it) + e] : 0.f;
    }
  };
#pragma unroll
  for (int a = 0; a < SCAN_AHEAD; ++a) load(a, buf[a], hbuf[a]);
  for (int it = 0; it < nc; ++it) {
    const int c = chunk(it);
    const int64_t base = slot(it);
    const float decay = __expf(send[(static_cast<int64_t>(bi) * nc + c) * H + h]);
    float cur[SCAN_EPT], hcur[SCAN_EPT];
#pragma unroll
    for (int k = 0; k < SCAN_EPT; ++k) {
      cur[k] = buf[0][k];
      hcur[k] = hbuf[0][k];
#pragma unroll
      for (int a = 0; a + 1 < SCAN_AHEAD; ++a) {
        buf[a][k] = buf[a + 1][k];
        hbuf[a][k] = hbuf[a + 1][k];
      }
    }
    load(it + SCAN_AHEAD, buf[SCAN_AHEAD - 1], hbuf[SCAN_AHEAD - 1]);
    float gh = 0.f;
#pragma unroll
    for (int k = 0; k < SCAN_EPT; ++k) {
      const int e = tid + SCAN_THREADS * k;
      if (e < nvalid) {
        states[base + e] = run[k];
        if (REV) gh += run[k] * hcur[k];
      }
      run[k] = decay * run[k] + cur[k];
    }
    if (REV) {
      gh = wave_sum(gh);
      if (lane_id() == 0) sTmp[wave_id()] = gh;
      __syncthreads();
      if (tid == 0) {
        float t = 0.f;
#pragma unroll
        for (int q = 0; q < SCAN_THREADS / WAVE; ++q) t += sTmp[q];
        gh_part[((static_cast<int64_t>(bi) * nc + c) * H + h) * npb + pb] = t;
      }
      __syncthreads();
    }
  }
  if (last) {
#pragma unroll
    for (int k = 0; k < SCAN_EPT; ++k) {
      const int e = tid + SCAN_THREADS * k;
      if (e < nvalid) last[(static_cast<int64_t>(bi) * H + h) * PN + off0 + e] = run[k];
    }
  }
}

template <typename TX, typename TB, bool BF, bool REV>
static hipError_t launch_state(const Dims& d, const void* X, const void* Bm, const void* dt,
                               const float* A_log, const float* init, void* states, float* last,
                               const float* hstates, float* gh_part, float* send, hipStream_t st,
                               void* hbf = nullptr) {
  if constexpr (!BF) {
    // two passes: per-chunk sums in parallel, then the walk over chunks
    // half the d_state columns per workgroup when whole heads would leave
    // fewer than two workgroups per CU (the smaller problems)
    const int64_t units = static_cast<int64_t>(d.H) * d.nc() * d.b;
    if (units < 512 && d.N > NMAX / 2)
      hipLaunchKernelGGL((chunk_sum_f32_kernel<TX, TB, REV, 2>), dim3(2 * units), dim3(NTHREADS), 0, st,
                         static_cast<const TX*>(X), static_cast<const TB*>(Bm), static_cast<const TB*>(dt), A_log,
                         static_cast<float*>(states), send, d.T, d.H, d.P, d.N, d.G, d.Q);
    else
      hipLaunchKernelGGL((chunk_sum_f32_kernel<TX, TB, REV, 1>), dim3(units), dim3(NTHREADS), 0, st,
                         static_cast<const TX*>(X), static_cast<const TB*>(Bm), static_cast<const TB*>(dt), A_log,
                         static_cast<float*>(states), send, d.T, d.H, d.P, d.N, d.G, d.Q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(state_scan_kernel<REV>, dim3(state_npb(d) * d.H * d.b), dim3(SCAN_THREADS), 0, st,
                       static_cast<float*>(states), send, init, last, hstates, gh_part, d.nc(), d.H, d.P, d.N);
    return hipGetLastError();
  } else {
    dim3 grid(state_npb(d) * d.H * d.b);
    hipLaunchKernelGGL((chunk_state_kernel<TX, TB, TB, BF, REV>), grid, dim3(NTHREADS), 0, st,
                       static_cast<const TX*>(X), static_cast<const TB*>(Bm), static_cast<const TB*>(dt),
                       A_log, init, states, last, hstates, gh_part, static_cast<uint16_t*>(hbf), d.T, d.H,
                       d.P, d.N, d.G, d.Q);
    return hipGetLastError();
  }
}

hipError_t launch_chunk_state_fwd(const Dims& d, DType act, const void* x, const void* B,
                                  const void* dt, const float* A_log, const float* init,
                                  float* states, float* final_state, void* hbf, float* send, hipStream_t st) {
  if (act == BF16)
    return launch_state<uint16_t, uint16_t, true, false>(d, x, B, dt, A_log, init, states, final_state,
                                                         nullptr, nullptr, send, st, hbf);
  return launch_state<float, float, false, false>(d, x, B, dt, A_log, init, states, final_state, nullptr,
                                                  nullptr, send, st);
}

hipError_t launch_chunk_state_bwd(const Dims& d, DType act, DType dyt, const void* dy,
                                  const void* C, const void* dt, const float* A_log, const float* dfinal,
                                  const float* states, void* gamma, float* dinit, float* gh_part,
                                  void* hbf, float* send, hipStream_t st) {
  if (act == BF16) {
    if (dyt == BF16)
      return launch_state<uint16_t, uint16_t, true, true>(d, dy, C, dt, A_log, dfinal, gamma, dinit,
                                                          states, gh_part, send, st, hbf);
    return launch_state<float, uint16_t, true, true>(d, dy, C, dt, A_log, dfinal, gamma, dinit, states,
                                                     gh_part, send, st, hbf);
  }
  if (dyt == BF16)
    return launch_state<uint16_t, float, false, true>(d, dy, C, dt, A_log, dfinal, gamma, dinit, states,
                                                      gh_part, send, st);
  return launch_state<float, float, false, true>(d, dy, C, dt, A_log, dfinal, gamma, dinit, states,
                                                 gh_part, send, st);
}

}  // namespace ssd
