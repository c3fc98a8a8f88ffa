/*
 * C ABI of the MI355X (gfx950) Mamba-2 SSD library: the SSD core forward and
 * analytic backward, plus the block-shell ops around it (causal depthwise
 * conv1d + SiLU, RMSNorm-gated output).
 *
 * The operations are those of the burn_dragon_kernel 0.5.0 page
 * "src/sequence/mamba2/backward.rs":
 *   ssd_fwd   the recurrence of ssd_forward_state_history_reference
 *             h_t = exp(dt_t A_h) h_{t-1} + dt_t x_t (outer) B_t, A_h = -exp(A_log_h),
 *             and the readout y_t = C_t . h_t + D_h x_t of the block backward
 *             (the y_grouped expression); head h reads group h / (nheads/ngroups).
 *   ssd_bwd   the gradients of ssd_backward_reference (grad_x, grad_b, grad_c,
 *             grad_dt, grad_a_log, grad_d_skip) plus the gradient of the initial
 *             state, for the loss sum(dy * y).  The optional saved state history
 *             and the "recompute" mode mirror the fused backward's optional
 *             ssd_state_history argument (its two parity tests).
 *   mamba2_conv1d_silu_*      depthwise_conv_preact_with_history + silu, and the
 *                             block backward's conv / SiLU tap loop.
 *   mamba2_rmsnorm_gated_*    rmsnorm_gated_{forward,backward}_from_inv_rms with
 *                             inv_rms = 1/sqrt(mean(y^2) + eps).
 *   ssd_dt_softplus_*         dt = softplus(dt_raw + dt_bias) in front of the core
 *                             and its gradient (dt_pre, grad_dt_pre, grad_dt_bias).
 *
 * Conventions (all entry points):
 *  - Every tensor pointer is a DEVICE pointer owned by the caller; the library
 *    never allocates, frees or keeps them.  Scratch memory is the caller's
 *    `workspace` (size from the matching *_workspace_bytes call).
 *  - Layouts are row-major and contiguous.  bf16 tensors hold raw bfloat16 bits.
 *  - Every output is overwritten (never accumulated into).
 *  - `stream` is a hipStream_t (0 = the null stream).  Work is enqueued
 *    asynchronously; the call returns once it is enqueued.
 *  - Arguments are checked before anything is enqueued; on failure nothing is
 *    enqueued and the call returns a negative ssd_status, with a description in
 *    ssd_last_error() (thread-local, valid until the next call on that thread).
 *    A launch failure returns SSD_ERR_HIP naming the kernel.
 *  - Tensor pointers must be 16-byte aligned (SSD_ERR_ALIGN otherwise).
 *  - Results are deterministic: every reduction runs in a fixed order.
 *  - Calls that share a workspace must be ordered on one stream.
 */
#ifndef SSD_MI355X_H
#define SSD_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSD_OK = 0,
  SSD_ERR_INVALID_ARG = -1, /* null required pointer, non-positive size */
  SSD_ERR_SHAPE = -2,       /* unsupported or inconsistent dimensions */
  SSD_ERR_DTYPE = -3,       /* unknown dtype code */
  SSD_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
  SSD_ERR_HIP = -5,         /* a HIP launch failed */
  SSD_ERR_ALIGN = -6        /* a tensor pointer is not 16-byte aligned */
} ssd_status;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

/* The statement of one SSD problem (the page's batch, time, nheads, headdim,
 * d_state, ngroups, plus the chunk length of the chunked algorithm).
 * Limits: 1 <= headdim <= 64, 1 <= dstate <= 128, 1 <= chunk <= 256,
 * seqlen % chunk == 0, nheads % ngroups == 0, nheads <= 65535,
 * batch <= 65535.  batch == 0 or seqlen == 0 is an empty problem. */
typedef struct {
  int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk;
  int32_t act_dtype; /* dtype of x, dt, B, C and y (ssd_dtype) */
  int32_t dy_dtype;  /* dtype of dy (ssd_dtype) */
} ssd_problem;

/* Bytes of workspace ssd_fwd (for_backward = 0) or ssd_bwd (for_backward = 1)
 * needs.  has_chunk_states tells whether the caller passes chunk_states (fwd:
 * as an output, bwd: as the saved history); without them the library keeps
 * the chunk states in the workspace.  bf16 problems (headdim and dstate
 * multiples of 8) also keep a bf16 copy of the chunk states there, and every
 * problem keeps a [b, nc, H] f32 array of per-chunk decays, so a workspace is
 * needed even when chunk_states is given.  Returns 0 for an invalid or empty
 * problem. */
size_t ssd_workspace_bytes(const ssd_problem* prob, int for_backward, int has_chunk_states);

/* Forward.
 *   x [b,T,H,P], dt [b,T,H] (dt after softplus, > 0), B, C [b,T,G,N]: act_dtype
 *   A_log, D [H]: f32
 *   init_state [b,H,P,N] f32, nullable (zeros)
 *   y [b,T,H,P] act_dtype (output)
 *   final_state [b,H,P,N] f32, nullable (output): state after the last step
 *   chunk_states [b,T/chunk,H,P,N] f32, nullable (output): the state entering
 *     each chunk (chunk 0: init_state) = the page's per-step state history
 *     sampled at the last step of the previous chunk.  Pass it to ssd_bwd to
 *     skip the recomputation. */
int ssd_fwd(const ssd_problem* prob, const void* x, const void* dt, const float* A_log,
            const void* B, const void* C, const float* D, const float* init_state, void* y,
            float* final_state, float* chunk_states, void* workspace, size_t workspace_bytes,
            void* stream);

/* ssd_fwd with a bf16 copy of the chunk states as a second, optional output
 * (the same recurrence and reference as ssd_fwd).
 *   chunk_states_bf16 [b,T/chunk,H,P,N] bf16 (round to nearest even of the
 *     f32 states), nullable (output).  Only for problems the bf16 kernels run
 *     (act_dtype SSD_BF16, headdim and dstate multiples of 8; SSD_ERR_INVALID_ARG
 *     otherwise).  Half the size of chunk_states and all that the bf16
 *     backward reads of the history: pass it to ssd_bwd_ex.
 * Other arguments, results and errors as for ssd_fwd (ssd_fwd is this call
 * with chunk_states_bf16 = NULL). */
int ssd_fwd_ex(const ssd_problem* prob, const void* x, const void* dt, const float* A_log,
               const void* B, const void* C, const float* D, const float* init_state, void* y,
               float* final_state, float* chunk_states, void* chunk_states_bf16, void* workspace,
               size_t workspace_bytes, void* stream);

/* Backward of L = sum(dy * y) + sum(d_final_state * final_state).
 *   inputs as in ssd_fwd; dy [b,T,H,P] in dy_dtype
 *   d_final_state [b,H,P,N] f32, nullable (zeros): the gradient reaching the
 *     state after the last step, so that consecutive segments of a sequence
 *     can chain their backward passes (it starts the reverse state pass)
 *   chunk_states: nullable; when given it must be what ssd_fwd wrote for the
 *     same inputs (not checked); when null the states are recomputed
 *   outputs (f32, all required except d_init_state):
 *     dx [b,T,H,P], ddt [b,T,H], dA_log [H], dB, dC [b,T,G,N], dD [H]
 *     d_init_state [b,H,P,N] nullable: gradient of the initial state (written
 *     also when init_state is null: the gradient at a zero initial state). */
int ssd_bwd(const ssd_problem* prob, const void* x, const void* dt, const float* A_log,
            const void* B, const void* C, const float* D, const float* init_state,
            const float* chunk_states, const void* dy, const float* d_final_state, float* dx,
            float* ddt, float* dA_log, float* dB, float* dC, float* dD, float* d_init_state,
            void* workspace, size_t workspace_bytes, void* stream);

/* ssd_bwd taking the saved history in bf16 (the same gradients and reference
 * as ssd_bwd).
 *   chunk_states_bf16: nullable; when given it must be what ssd_fwd_ex wrote
 *     for the same inputs (not checked), and only for problems the bf16
 *     kernels run (act_dtype and dy_dtype SSD_BF16, headdim and dstate
 *     multiples of 8; SSD_ERR_INVALID_ARG otherwise).  The fused bf16
 *     backward then reads no f32 states (chunk_states may be NULL, and is
 *     not read if given); the split form (SSD_BF16_BWD=split) ignores it and
 *     uses chunk_states or recomputes.  The bf16 backward reads the states
 *     only in bf16 in either case (its inner product <Gamma, H_c> and the
 *     readout term take the bf16 copy).
 * ssd_workspace_bytes(prob, 1, 0) is enough when only chunk_states_bf16 is
 * given.  Other arguments, results and errors as for ssd_bwd (ssd_bwd is
 * this call with chunk_states_bf16 = NULL). */
int ssd_bwd_ex(const ssd_problem* prob, const void* x, const void* dt, const float* A_log,
               const void* B, const void* C, const float* D, const float* init_state,
               const float* chunk_states, const void* chunk_states_bf16, const void* dy,
               const float* d_final_state, float* dx, float* ddt, float* dA_log, float* dB, float* dC,
               float* dD, float* d_init_state, void* workspace, size_t workspace_bytes, void* stream);

/* ssd_bwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results and errors as ssd_bwd, without the workspace: the
 * scratch comes from a library-owned device array of SSD_NOALLOC_SCRATCH_BYTES
 * on each GPU (held from the first call on that GPU until the process ends).
 * Problems whose ssd_workspace_bytes(prob, 1, chunk_states != NULL) exceeds
 * it are rejected with SSD_ERR_WORKSPACE.  The call allocates nothing: no
 * hipMalloc, hipFree or allocating library routine.  Every call on one GPU
 * uses that GPU's one array, so calls that overlap on a GPU (different
 * streams, or threads, without ordering between them) race; order them on one
 * stream.  The stream must belong to the current device (SSD_ERR_INVALID_ARG
 * otherwise). */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int ssd_bwd_noalloc(const ssd_problem* prob, const void* x, const void* dt, const float* A_log,
                    const void* B, const void* C, const float* D, const float* init_state,
                    const float* chunk_states, const void* dy, const float* d_final_state, float* dx,
                    float* ddt, float* dA_log, float* dB, float* dC, float* dD, float* d_init_state,
                    void* stream);

/* Causal depthwise conv1d (zero initial state) followed by SiLU, split into
 * the SSD inputs.  xbc [b,T,conv_dim] with conv_dim = d_inner + 2*ngroups*dstate
 * (channel order: x, then B, then C); w [conv_dim, d_conv] f32, tap d_conv-1
 * multiplies the current step; bias [conv_dim] f32.  Outputs in `dtype`:
 * x_out [b,T,d_inner], B_out, C_out [b,T,ngroups,dstate].  1 <= d_conv <= 8. */
int mamba2_conv1d_silu_fwd(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t ngroups,
                           int64_t dstate, int64_t d_conv, int32_t dtype, const void* xbc,
                           const float* w, const float* bias, void* x_out, void* B_out,
                           void* C_out, void* stream);

size_t mamba2_conv1d_silu_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner,
                                              int64_t ngroups, int64_t dstate, int64_t d_conv);

/* Backward of mamba2_conv1d_silu_fwd.  dx [b,T,d_inner], dB, dC [b,T,G,N] are
 * the f32 gradients of its three outputs.  Outputs: dxbc, b*T rows of
 * conv_dim elements, dxbc_ld elements apart (0 or conv_dim: packed; else a
 * multiple of 4 above conv_dim, e.g. to leave room for the dt_raw gradient
 * beside it as one GEMM operand), in `dxbc_dtype` (SSD_F32, or SSD_BF16 rounded to nearest
 * even: the values an f32 -> bf16 cast of the f32 output gives); dw
 * [conv_dim,d_conv] and dbias [conv_dim] f32. */
int mamba2_conv1d_silu_bwd(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t ngroups,
                           int64_t dstate, int64_t d_conv, int32_t dtype, const void* xbc,
                           const float* w, const float* bias, const float* dx, const float* dB,
                           const float* dC, int32_t dxbc_dtype, void* dxbc, int64_t dxbc_ld,
                           float* dw, float* dbias, void* workspace, size_t workspace_bytes,
                           void* stream);

/* RMSNorm-gated forward over rows of `width`: inv_rms = 1/sqrt(mean(y^2)+eps),
 * out = y * inv_rms * w * silu(z).  y, z, out in `dtype`; w [width] f32;
 * inv_rms [rows] f32 (output, saved for the backward). */
int mamba2_rmsnorm_gated_fwd(int64_t rows, int64_t width, float eps, int32_t dtype, const void* y,
                             const void* z, const float* w, void* out, float* inv_rms,
                             void* stream);

size_t mamba2_rmsnorm_gated_bwd_workspace_bytes(int64_t rows, int64_t width);

/* RMSNorm-gated backward with the saved inv_rms.  g [rows,width] is the
 * gradient of `out` in `g_dtype`.  Outputs: dy [rows,width] in `dy_dtype`
 * (SSD_F32, or SSD_BF16 rounded to nearest even, e.g. to feed ssd_bwd's bf16
 * path as its dy); dz, rows of width elements dz_ld apart (0 or width:
 * packed; else a multiple of 8 above width, e.g. beside the other in_proj
 * gradients as one GEMM operand), in `dz_dtype` (likewise); dw [width] f32, a
 * fixed-order sum of per-64-row partials held in the workspace. */
int mamba2_rmsnorm_gated_bwd(int64_t rows, int64_t width, int32_t dtype, int32_t g_dtype,
                             int32_t dy_dtype, int32_t dz_dtype, const void* y, const void* z,
                             const float* w, const float* inv_rms, const void* g, void* dy, void* dz,
                             int64_t dz_ld, float* dw, void* workspace, size_t workspace_bytes,
                             void* stream);

/* dt activation in front of the core (burn_dragon_kernel src/sequence/mamba2/backward.rs,
 * tensorized_mamba2_backward_impl:
 * dt_pre = dt_raw + dt_bias, dt = softplus(dt_pre) with beta 1; after the fused
 * backward, grad_dt_pre = grad_dt * sigmoid(dt_pre) and grad_dt_bias is its sum
 * over batch and time).  Rows are the b*T steps of [b,T,nheads] arrays.
 *   ssd_dt_softplus_fwd: dt_raw, dt [rows,nheads] in `dtype` (bf16 output is
 *     rounded to nearest even, the form ssd_fwd / ssd_bwd read); dt_bias
 *     [nheads] f32.  dt may be passed to ssd_fwd and ssd_bwd as their dt.
 *   ssd_dt_softplus_bwd: ddt [rows,nheads] f32 is ssd_bwd's gradient of dt;
 *     outputs ddt_raw (the gradient of dt_raw, equal to that of dt_pre), rows
 *     of nheads elements ddt_raw_ld apart (0: nheads), in `ddt_raw_dtype`
 *     (SSD_F32, or SSD_BF16 rounded to nearest even), and f32 d_dt_bias
 *     [nheads], a fixed-order sum of per-64-row partials held in the
 *     workspace.
 * softplus(v) is evaluated as max(v,0) + log1p(exp(-|v|)).  Pointers are
 * 16-byte aligned device pointers; errors as for ssd_fwd. */
int ssd_dt_softplus_fwd(int64_t rows, int64_t nheads, int32_t dtype, const void* dt_raw,
                        const float* dt_bias, void* dt, void* stream);
size_t ssd_dt_softplus_bwd_workspace_bytes(int64_t rows, int64_t nheads);
int ssd_dt_softplus_bwd(int64_t rows, int64_t nheads, int32_t dtype, const void* dt_raw,
                        const float* dt_bias, const float* ddt, int32_t ddt_raw_dtype, void* ddt_raw,
                        int64_t ddt_raw_ld, float* d_dt_bias, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Plain GEMM for the input and output projections around the block slice
 * (the in_proj / out_proj products of a Mamba-2 block's forward and
 * backward): row-major C[m,n] = alpha * op(A) * op(B) + beta * C with bf16 A
 * and B, f32 accumulation, and C in c_dtype (SSD_F32 or SSD_BF16).  op(A) is
 * [m,k]: A stored [m,k], or [k,m] when trans_a != 0; op(B) is [k,n]: B stored
 * [k,n], or [n,k] when trans_b != 0.  lda, ldb, ldc are row strides in
 * elements.  Runs on the caller's stream through hipBLASLt (the fastest of
 * its heuristic's candidates for the shape, timed on the shape's first call,
 * which synchronises the stream and allocates a scratch output for the
 * trials), or rocBLAS gemm_ex where hipBLASLt offers no algorithm or
 * SSD_GEMM=rocblas is set.  Unlike the other entry points, the library
 * handles and the 128 MiB hipBLASLt workspace (one each per device, created on
 * first use) hold device memory of their own. */
int ssd_gemm(int32_t trans_a, int32_t trans_b, int64_t m, int64_t n, int64_t k, float alpha,
             const void* A, int64_t lda, const void* B, int64_t ldb, float beta, void* C,
             int32_t c_dtype, int64_t ldc, void* stream);

/* dst[i] = src[i] rounded to bf16 (nearest even), i < n: the f32 gradients of
 * the block slice cast for the bf16 projection GEMMs. */
int ssd_cast_f32_to_bf16(int64_t n, const float* src, void* dst, void* stream);

/* Description of the last failure on the calling thread ("" after success). */
const char* ssd_last_error(void);

/* Library version string. */
const char* ssd_version(void);

/* Opt-in per-kernel timing (a tracing aid, off by default).  ssd_profile_enable
 * clears earlier records and turns recording on (on != 0) or off.  While on,
 * every kernel an entry point launches is bracketed by two HIP events on the
 * caller's stream.  ssd_profile_kernel_ms waits for the recorded events and
 * returns the summed milliseconds and the number of launches of one kernel:
 * "chunk_state_fwd", "chunk_out_fwd", "chunk_state_fwd (recompute)",
 * "chunk_state_bwd", "chunk_bwd_col", "chunk_bwd_row", "bwd_dt", "bwd_split_sum",
 * "conv1d_silu_fwd", "conv1d_silu_bwd", "rmsnorm_gated_fwd",
 * "rmsnorm_gated_bwd", "dt_softplus_fwd", "dt_softplus_bwd".  Not for use
 * while other threads call the library. */
int ssd_profile_enable(int on);
/* Restrict recording to one kernel name (NULL or "" records every kernel), so
 * that the events of the others do not hold up the stream while one kernel is
 * timed.  Takes effect for launches made after the call. */
int ssd_profile_only(const char* kernel);
int ssd_profile_kernel_ms(const char* kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* SSD_MI355X_H */
