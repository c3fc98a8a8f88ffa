// Host-side launchers of the SSD kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

enum DType : int { F32 = 0, BF16 = 1 };

struct Dims {
  int b, T, H, P, N, G, Q;
  int nc() const { return T / Q; }
  int nb() const { return (Q + 63) / 64; }
  int hpg() const { return H / G; }
};

// Number of headdim rows one chunk-state workgroup owns.
constexpr int STATE_PB = 16;
inline int state_npb(const Dims& d) { return (d.P + STATE_PB - 1) / STATE_PB; }
// per-wave partials of <Gamma_{c+1}, H_c> that the fused backward kernel writes per (b, chunk, head)
constexpr int FUSED_GH_SLOTS = 8;
// the fused backward kernel's W area: per workgroup one 64 x 64 bf16 block of
// the head-summed W for each block pair (ib, j) below the diagonal
constexpr int FUSED_W_PAIR_BYTES = 64 * 64 * 2;
inline int fused_w_pairs(const Dims& d) { return d.nb() * (d.nb() - 1) / 2; }

// Forward state passing: states[b,c,h] = state entering chunk c, final = state
// after the last chunk.  `init` may be null (zero initial state), `final_state`
// may be null; hbf (nullable) receives the states rounded to bf16.
// send: [b, nc, H] floats of scratch (the f32 form writes each chunk's total
// log-decay there between its two passes).
hipError_t launch_chunk_state_fwd(const Dims& d, DType act, const void* x, const void* B,
                                  const void* dt, const float* A_log, const float* init,
                                  float* states, float* final_state, void* hbf, float* send, hipStream_t st);

// Reverse state-gradient pass: gamma[b,c,h] = gradient reaching the state that
// leaves chunk c, stored in the MFMA operand type (bf16 when act is BF16, else
// f32); dinit = gradient of the initial state (nullable);
// gh_part[b,c,h,pb] = partial <gamma[b,c,h], states[b,c,h]> over headdim block pb;
// hbf (nullable) = the states rounded to bf16, same layout.
hipError_t launch_chunk_state_bwd(const Dims& d, DType act, DType dyt, const void* dy,
                                  const void* C, const void* dt, const float* A_log, const float* dfinal,
                                  const float* states, void* gamma, float* dinit, float* gh_part,
                                  void* hbf, float* send, hipStream_t st);

// bf16 operands with asynchronous LDS staging (bwd_bf16_supported shapes):
// the chunk-state passes (same outputs as launch_chunk_state_fwd/_bwd) and the
// chunk output, which reads the bf16 copy of the states.
hipError_t launch_chunk_state_fwd_bf16(const Dims& d, const void* x, const void* B, const void* dt,
                                       const float* A_log, const float* init, float* states, float* final_state,
                                       void* hbf, hipStream_t st);
// counter (nullable): an arrival counter that the bf16 backward's fused kernel
// counts on, zeroed by this launch.
hipError_t launch_chunk_state_bwd_bf16(const Dims& d, const void* dy, const void* C, const void* dt,
                                       const float* A_log, const float* dfinal, const float* states, void* gamma,
                                       float* dinit, float* gh_part, void* hbf, unsigned* counter, hipStream_t st);
hipError_t launch_out_fwd_bf16(const Dims& d, int nsplit, const void* x, const void* B, const void* C,
                               const void* dt, const float* A_log, const float* D, const void* hbf, void* y,
                               hipStream_t st);

// paired: a workgroup takes row blocks nb - 1 - k and k of its chunk (grid
// b nc G nsplit ceil(nb / 2)); else one row block (grid b nc G nsplit nb).
hipError_t launch_chunk_out_fwd(const Dims& d, DType act, int nsplit, bool paired, const void* x, const void* B,
                                const void* C, const void* dt, const float* A_log, const float* D,
                                const float* states, void* y, hipStream_t st);

struct BwdScratch {
  float* rowM;   // [b,H,T] strictly-lower row sums of the decay-gradient matrix; with row_slots > 0,
                 // row_slots such arrays (slot jb: the part from 64-column block jb, rows of blocks >= jb)
  float* colE;   // [b,H,T] column sums (diagonal included) without the dt factor
  float* diagE;  // [b,H,T] diagonal entries
  float* Rp;     // [b,H,T] state-term of the dt gradient without the dt factor
  float* dsoff;  // [b,H,T] decay gradient from the incoming-state readout
  float* gh_part;  // [b,nc,H,npb] partial <Gamma_{c+1}, H_c> of the reverse chunk-state pass, or (fused
                   // kernel) [b,nc,H,FUSED_GH_SLOTS], one per wave of the fused kernel's workgroup
  float* dA_part;  // [b,nc,H]
  float* dD_part;  // [b,nc,nb,H]
  unsigned* done;  // one counter: the dt kernel's finished workgroups (zeroed by the row kernel)
  uint16_t* wstrips;  // fused kernel: [b,nc,G,nsplit][fused_w_pairs] blocks of FUSED_W_PAIR_BYTES
  float* dB_part;  // [nsplit,b,T,G,N] or null when nsplit == 1
  float* dC_part;
  int row_slots;      // 0: rowM holds the row sums; else the number of slots to add
  int64_t slot_elems;  // b * H * T: elements of one row-sum slot
};

// paired: a workgroup takes blocks k and nb - 1 - k of its chunk (grid
// b nc G nsplit ceil(nb / 2)); else one block (grid b nc G nsplit nb).
hipError_t launch_chunk_bwd_col(const Dims& d, DType act, DType dyt, int nsplit, bool paired, const void* x,
                                const void* B, const void* C, const void* dt, const void* dy,
                                const float* A_log, const float* D, const void* gamma, float* dx,
                                float* dB_out, const BwdScratch& s, hipStream_t st);

hipError_t launch_chunk_bwd_row(const Dims& d, DType act, DType dyt, int nsplit, bool paired, const void* x,
                                const void* B, const void* C, const void* dt, const void* dy,
                                const float* A_log, const float* states, float* dC_out,
                                const BwdScratch& s, hipStream_t st);

// bf16 operands (activations and dy) with asynchronous LDS staging: headdim
// and d_state multiples of 8 and tile offsets within 1 GiB.
bool bwd_bf16_supported(const Dims& d);
hipError_t launch_bwd_row_bf16(const Dims& d, int nsplit, const void* x, const void* B, const void* C,
                               const void* dt, const void* dy, const float* A_log, const void* hbf,
                               float* dC_out, const BwdScratch& s, hipStream_t st);
hipError_t launch_bwd_col_bf16(const Dims& d, int nsplit, const void* x, const void* B, const void* C,
                               const void* dt, const void* dy, const float* A_log, const float* D,
                               const void* gamma, float* dx, float* dB_out, const BwdScratch& s,
                               hipStream_t st);

// The column and row work of the bf16 kernels in one kernel (ssd_bwd_fused.hip):
// one workgroup per (batch, chunk, group, head split); dx, dB and dC (or the
// head-split partials), the per-column sums, the readout term, dD partials,
// and the row sums of M in s.row_slots = nb slots; then, per workgroup, ddt of
// its heads and chunk, and in the last workgroup to finish dA_log and dD (the
// dt kernel's work).  Reads the bf16 copy of the states (hbf), Gamma and
// s.gh_part; needs s.done zeroed by an earlier launch on the stream (the
// reverse chunk-state kernel does it) and leaves it zero.
hipError_t launch_bwd_fused_bf16(const Dims& d, int nsplit, const void* x, const void* B, const void* C,
                                 const void* dt, const void* dy, const float* A_log, const float* D,
                                 const void* gamma, const void* hbf, float* dx, float* dB_out, float* dC_out,
                                 float* ddt, float* dA_log, float* dD, const BwdScratch& s, hipStream_t st);

// dt gradient per token, and dA_log and dD (fixed-order sums of the per-chunk
// partials, taken by the launch's last workgroup).  Needs s.done zeroed by an
// earlier launch on the stream (the row kernel does it).
hipError_t launch_bwd_dt(const Dims& d, DType act, const void* dt, const float* A_log, float* ddt, float* dA_log,
                         float* dD, const BwdScratch& s, hipStream_t st);

// dB and dC as sums of the head-split partials (nothing to do when nsplit == 1).
hipError_t launch_bwd_split_sum(const Dims& d, int nsplit, float* dB, float* dC, const BwdScratch& s,
                                hipStream_t st);

// Writes `value` into n floats (used for empty problems).
hipError_t launch_fill(float* p, int64_t n, float value, hipStream_t st);
hipError_t launch_copy(float* dst, const float* src, int64_t n, hipStream_t st);

}  // namespace ssd
