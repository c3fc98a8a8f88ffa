// C ABI of the SSD library: argument checks, workspace plan and the launch
// sequence of every entry point declared in include/ssd.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdlib>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/ssd.h"
#include "ssd_common.hpp"
#include "gemm_launch.hpp"
#include "shell_launch.hpp"
#include "ssd_launch.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return SSD_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool valid_dtype(int32_t t) { return t == SSD_F32 || t == SSD_BF16; }

// Checks the problem statement; fills `d` on success.
int check_problem(const ssd_problem* p, ssd::Dims* d) {
  if (!p) return fail(SSD_ERR_INVALID_ARG, "problem is null");
  if (!valid_dtype(p->act_dtype)) return fail(SSD_ERR_DTYPE, "act_dtype %d is not SSD_F32 or SSD_BF16", p->act_dtype);
  if (!valid_dtype(p->dy_dtype)) return fail(SSD_ERR_DTYPE, "dy_dtype %d is not SSD_F32 or SSD_BF16", p->dy_dtype);
  if (p->batch < 0 || p->seqlen < 0)
    return fail(SSD_ERR_INVALID_ARG, "batch (%lld) and seqlen (%lld) must be >= 0", (long long)p->batch,
                (long long)p->seqlen);
  if (p->nheads <= 0 || p->headdim <= 0 || p->dstate <= 0 || p->ngroups <= 0 || p->chunk <= 0)
    return fail(SSD_ERR_INVALID_ARG, "nheads, headdim, dstate, ngroups and chunk must be > 0");
  if (p->headdim > ssd::PMAX)
    return fail(SSD_ERR_SHAPE, "headdim %lld exceeds the supported maximum %d", (long long)p->headdim, ssd::PMAX);
  if (p->dstate > ssd::NMAX)
    return fail(SSD_ERR_SHAPE, "dstate %lld exceeds the supported maximum %d", (long long)p->dstate, ssd::NMAX);
  if (p->chunk > ssd::QMAX)
    return fail(SSD_ERR_SHAPE, "chunk %lld exceeds the supported maximum %d", (long long)p->chunk, ssd::QMAX);
  if (p->nheads % p->ngroups)
    return fail(SSD_ERR_SHAPE, "nheads %lld is not a multiple of ngroups %lld", (long long)p->nheads,
                (long long)p->ngroups);
  if (p->seqlen % p->chunk)
    return fail(SSD_ERR_SHAPE, "seqlen %lld is not a multiple of chunk %lld", (long long)p->seqlen,
                (long long)p->chunk);
  if (p->nheads > 65535 || p->batch > 65535)
    return fail(SSD_ERR_SHAPE, "nheads and batch must be <= 65535");
  const int64_t elems = p->batch * p->seqlen * p->nheads * p->headdim;
  if (p->seqlen > (int64_t(1) << 30) || elems > (int64_t(1) << 40))
    return fail(SSD_ERR_SHAPE, "problem too large");
  // The largest launch grids: one workgroup per (batch, chunk, head, 64-row
  // block) at most (general kernels, groups split down to single heads), one
  // per 256 elements of dB / dC (head-split sums) and of the [b, T, H] dt
  // series.  Each must fit a one-dimensional grid.
  const int64_t nchunks = p->seqlen / p->chunk, nblocks = (p->chunk + 63) / 64;
  const int64_t grid_max = (int64_t(1) << 31) - 1;
  if (p->batch * nchunks * p->nheads * nblocks > grid_max ||
      (p->batch * p->seqlen * p->ngroups * p->dstate + 255) / 256 > grid_max ||
      (p->batch * p->seqlen * p->nheads + 255) / 256 > grid_max)
    return fail(SSD_ERR_SHAPE, "problem too large: a launch grid would exceed %lld workgroups",
                (long long)grid_max);
  d->b = static_cast<int>(p->batch);
  d->T = static_cast<int>(p->seqlen);
  d->H = static_cast<int>(p->nheads);
  d->P = static_cast<int>(p->headdim);
  d->N = static_cast<int>(p->dstate);
  d->G = static_cast<int>(p->ngroups);
  d->Q = static_cast<int>(p->chunk);
  return SSD_OK;
}

// Heads of a group are split over this many workgroups so that one launch has
// at least `target` workgroups (never more splits than heads per group).  The
// bf16 kernels give one workgroup two 64-row blocks of a chunk (paired so that
// every workgroup has the same work), the general ones one block.
int choose_nsplit_base(const ssd::Dims& d, int64_t target, int64_t base) {
  const int hpg = d.hpg();
  for (int s = 1; s <= hpg; ++s)
    if (hpg % s == 0 && base * s >= target) return s;
  return hpg;
}
int choose_nsplit(const ssd::Dims& d, int64_t target, bool paired) {
  const int64_t base = static_cast<int64_t>(d.b) * d.nc() * d.G * (paired ? (d.nb() + 1) / 2 : d.nb());
  const int hpg = d.hpg();
  for (int s = 1; s <= hpg; ++s)
    if (hpg % s == 0 && base * s >= target) return s;
  return hpg;
}
constexpr int64_t kFwdTarget = 512;
constexpr int64_t kBwdTarget = 256;
// The general forward kernel forms C.B^T once per workgroup for all of its
// heads.  Splitting a group's heads down to one or two per workgroup repeats
// that product for every head, so then it splits only until the grid fills the
// CUs once (measured: 24 heads per group, 1 -> 3 heads per workgroup,
// 0.128 -> 0.088 ms; with 64 heads, 32 per workgroup in two rounds stays 4 %
// faster than 64 in one).
int general_fwd_nsplit(const ssd::Dims& d) {
  const int s = choose_nsplit(d, kFwdTarget, false);
  return d.hpg() / s >= 3 ? s : choose_nsplit(d, kBwdTarget, false);
}
// Paired row blocks (nb - 1 - k and k in one workgroup) give every workgroup
// the same work, but half the workgroups: taken when the paired grid still
// fills the CUs once with at least three heads per workgroup (long workload,
// 64 heads: 256 workgroups of 32 heads and two blocks instead of 512 of 32
// heads and one); the split is then the smallest that does.
// The same choice for the general backward's column and row kernels.
struct GeneralShape {
  int nsplit;
  bool paired;
};
int general_paired_nsplit(const ssd::Dims& d) {
  const int64_t base = static_cast<int64_t>(d.b) * d.nc() * d.G * ((d.nb() + 1) / 2);
  const int hpg = d.hpg();
  if (d.nb() > 1)
    for (int s = 1; s <= hpg / 3; ++s)
      if (hpg % s == 0 && base * s >= kBwdTarget) return s;
  return 0;
}
GeneralShape general_fwd_shape(const ssd::Dims& d) {
  const int s = general_paired_nsplit(d);
  return s ? GeneralShape{s, true} : GeneralShape{general_fwd_nsplit(d), false};
}

struct FwdPlan {
  size_t states = 0, hbf = 0, send = 0, total = 0;
  bool bf16 = false;  // bf16 output kernel with asynchronous staging (reads a bf16 copy of the states)
};
struct BwdPlan {
  size_t states = 0, gamma = 0, hbf = 0, gh = 0, rowM = 0, colE = 0, diagE = 0, Rp = 0, dsoff = 0, dA = 0, dD = 0,
         done = 0, wst = 0, dB = 0, dC = 0, send = 0, total = 0;
  int nsplit = 1;
  bool paired = false;  // general column and row kernels: two row blocks per workgroup
  bool bf16 = false;   // bf16 kernels with asynchronous staging (they also need a bf16 copy of the states)
  bool fused = false;  // the bf16 column and row work in one kernel (row sums of M in nb slots)
};

// The bf16 backward runs the fused column-and-row kernel unless SSD_BF16_BWD=split
// selects the separate column and row kernels (kept for comparison).
bool bf16_bwd_fused() {
  static const bool fused = [] {
    const char* v = std::getenv("SSD_BF16_BWD");
    return !(v && std::strcmp(v, "split") == 0);
  }();
  return fused;
}

size_t state_bytes(const ssd::Dims& d) {
  return sizeof(float) * static_cast<size_t>(d.b) * d.nc() * d.H * d.P * d.N;
}

bool use_bf16_kernels(const ssd::Dims& d, int act, int dyt) {
  return act == SSD_BF16 && dyt == SSD_BF16 && ssd::bwd_bf16_supported(d);
}

FwdPlan plan_fwd(const ssd::Dims& d, bool has_states, bool bf16) {
  FwdPlan p;
  p.bf16 = bf16;
  size_t off = 0;
  // the bf16 family's output kernel reads the bf16 copy of the states, so
  // the f32 ones are written only when the caller asks for them
  if (!has_states && !bf16) {
    p.states = off;
    off += align_up(state_bytes(d));
  }
  if (bf16) {
    p.hbf = off;
    off += align_up(state_bytes(d) / 2);
  }
  p.send = off;  // per-chunk total log-decay of the two-pass f32 chunk-state form
  off += align_up(sizeof(float) * static_cast<size_t>(d.b) * d.nc() * d.H);
  p.total = off;
  return p;
}

BwdPlan plan_bwd(const ssd::Dims& d, bool has_states, bool bf16) {
  BwdPlan p;
  p.bf16 = bf16;
  p.fused = bf16 && bf16_bwd_fused();
  // the fused kernel takes one workgroup per (batch, chunk, group) and head split
  p.nsplit = p.fused ? choose_nsplit_base(d, kBwdTarget, static_cast<int64_t>(d.b) * d.nc() * d.G)
                     : choose_nsplit(d, kBwdTarget, bf16);
  if (!bf16) {
    const int s = general_paired_nsplit(d);
    if (s) p.nsplit = s, p.paired = true;
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const size_t bht = sizeof(float) * static_cast<size_t>(d.b) * d.H * d.T;
  // the fused form reads only the bf16 copy of the states (recomputed into
  // hbf when no history is given); the others need the f32 states
  if (!has_states && !p.fused) p.states = take(state_bytes(d));
  p.gamma = take(state_bytes(d));
  if (bf16) p.hbf = take(state_bytes(d) / 2);
  p.gh = take(sizeof(float) * static_cast<size_t>(d.b) * d.nc() * d.H *
              (p.fused ? ssd::FUSED_GH_SLOTS : ssd::state_npb(d)));
  p.rowM = take(p.fused ? bht * d.nb() : bht);
  p.colE = take(bht);
  p.diagE = take(bht);
  p.Rp = take(bht);
  p.dsoff = take(bht);
  p.dA = take(sizeof(float) * static_cast<size_t>(d.b) * d.nc() * d.H);
  p.dD = take(sizeof(float) * static_cast<size_t>(d.b) * d.nc() * d.nb() * d.H);
  p.done = take(sizeof(unsigned));
  p.send = take(sizeof(float) * static_cast<size_t>(d.b) * d.nc() * d.H);
  if (p.fused)
    p.wst = take(static_cast<size_t>(d.b) * d.nc() * d.G * p.nsplit * ssd::fused_w_pairs(d) *
                 ssd::FUSED_W_PAIR_BYTES);
  if (p.nsplit > 1) {
    const size_t part = sizeof(float) * static_cast<size_t>(p.nsplit) * d.b * d.T * d.G * d.N;
    p.dB = take(part);
    p.dC = take(part);
  }
  p.total = off;
  return p;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SSD_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
}

// Opt-in per-kernel timing: when enabled, every launch made by an entry point
// is bracketed by two HIP events recorded on the caller's stream.
struct ProfRecord {
  const char* name;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::string g_prof_only;  // record this kernel only (empty: every kernel)
std::vector<ProfRecord> g_prof_records;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  // timing only: no system-scope fence (a cache write-back and invalidate at
  // each record, which otherwise holds up the next kernel); the events are
  // read after the caller has synchronised the stream
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// Set while ssd_bwd_noalloc runs: its launches record no events (creating one
// is an allocation of the runtime's).
thread_local bool g_prof_suppress = false;

hipEvent_t prof_begin(hipStream_t st, const char* name) {
  if (g_prof_suppress) return nullptr;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on || (!g_prof_only.empty() && g_prof_only != name)) return nullptr;
  hipEvent_t e = prof_event();
  if (e && hipEventRecord(e, st) != hipSuccess) return nullptr;
  return e;
}

void prof_end(hipEvent_t start, const char* name, hipStream_t st) {
  if (!start) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  hipEvent_t e = prof_event();
  if (e && hipEventRecord(e, st) == hipSuccess) g_prof_records.push_back({name, start, e});
}

#define SSD_LAUNCH(expr, what)                                \
  do {                                                        \
    hipEvent_t p_ = prof_begin(st, what);                     \
    hipError_t e_ = (expr);                                   \
    if (e_ != hipSuccess) return hip_fail(e_, what);          \
    prof_end(p_, what, st);                                   \
  } while (0)

}  // namespace

extern "C" {

const char* ssd_last_error(void) { return g_last_error.c_str(); }

const char* ssd_version(void) { return "ssd-mi355x 0.1 (gfx950)"; }

int ssd_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (const ProfRecord& r : g_prof_records) {
    g_prof_pool.push_back(r.start);
    g_prof_pool.push_back(r.stop);
  }
  g_prof_records.clear();
  g_prof_on = on != 0;
  return ok();
}

int ssd_profile_only(const char* kernel) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_only = kernel ? kernel : "";
  return ok();
}

int ssd_profile_kernel_ms(const char* kernel, double* total_ms, int64_t* launches) {
  if (!kernel || !total_ms || !launches) return fail(SSD_ERR_INVALID_ARG, "ssd_profile_kernel_ms: null argument");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  double tot = 0.0;
  int64_t n = 0;
  for (const ProfRecord& r : g_prof_records) {
    if (std::strcmp(r.name, kernel) != 0) continue;
    hipError_t e = hipEventSynchronize(r.stop);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return hip_fail(e, "profile event");
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return ok();
}

size_t ssd_workspace_bytes(const ssd_problem* prob, int for_backward, int has_chunk_states) {
  ssd::Dims d;
  if (check_problem(prob, &d) != SSD_OK) return 0;
  if (d.b == 0 || d.T == 0) return 0;
  return for_backward ? plan_bwd(d, has_chunk_states != 0, use_bf16_kernels(d, prob->act_dtype, prob->dy_dtype)).total
                      : plan_fwd(d, has_chunk_states != 0, use_bf16_kernels(d, prob->act_dtype, prob->act_dtype)).total;
}

int ssd_fwd(const ssd_problem* prob, const void* x, const void* dt, const float* A_log, const void* B,
            const void* C, const float* D, const float* init_state, void* y, float* final_state,
            float* chunk_states, void* workspace, size_t workspace_bytes, void* stream) {
  return ssd_fwd_ex(prob, x, dt, A_log, B, C, D, init_state, y, final_state, chunk_states, nullptr, workspace,
                    workspace_bytes, stream);
}

int ssd_fwd_ex(const ssd_problem* prob, const void* x, const void* dt, const float* A_log, const void* B,
               const void* C, const float* D, const float* init_state, void* y, float* final_state,
               float* chunk_states, void* chunk_states_bf16, void* workspace, size_t workspace_bytes,
               void* stream) {
  ssd::Dims d;
  int rc = check_problem(prob, &d);
  if (rc != SSD_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const ssd::DType act = static_cast<ssd::DType>(prob->act_dtype);
  if (!A_log || !D) return fail(SSD_ERR_INVALID_ARG, "ssd_fwd: A_log and D are required");
  const bool empty = d.b == 0 || d.T == 0;
  if (!empty && (!x || !dt || !B || !C || !y))
    return fail(SSD_ERR_INVALID_ARG, "ssd_fwd: x, dt, B, C and y are required");
  if (chunk_states_bf16 && !use_bf16_kernels(d, prob->act_dtype, prob->act_dtype))
    return fail(SSD_ERR_INVALID_ARG,
                "ssd_fwd: chunk_states_bf16 needs a problem the bf16 kernels run (bf16 activations, headdim and "
                "dstate multiples of 8)");
  const void* ptrs[] = {x, dt, A_log, B, C, D, init_state, y, final_state, chunk_states, chunk_states_bf16};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(SSD_ERR_ALIGN, "ssd_fwd: a tensor pointer is not 16-byte aligned");
  const int64_t state_elems = static_cast<int64_t>(d.b) * d.H * d.P * d.N;
  if (empty) {
    if (final_state) {
      if (init_state)
        SSD_LAUNCH(ssd::launch_copy(final_state, init_state, state_elems, st), "copy");
      else
        SSD_LAUNCH(ssd::launch_fill(final_state, state_elems, 0.f, st), "fill");
    }
    return ok();
  }
  const FwdPlan plan = plan_fwd(d, chunk_states != nullptr, use_bf16_kernels(d, prob->act_dtype, prob->act_dtype));
  if (!workspace) return fail(SSD_ERR_WORKSPACE, "ssd_fwd: workspace is null (%zu bytes needed)", plan.total);
  if (workspace_bytes < plan.total)
    return fail(SSD_ERR_WORKSPACE, "ssd_fwd: workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
                plan.total);
  if (workspace && !aligned16(workspace)) return fail(SSD_ERR_ALIGN, "ssd_fwd: workspace is not 16-byte aligned");
  // bf16 family: f32 states only when asked for, the bf16 copy (read by the
  // output kernel) into the caller's buffer when given
  float* states = chunk_states ? chunk_states : plan.bf16 ? nullptr : at<float>(workspace, plan.states);
  void* hbf = plan.bf16 ? (chunk_states_bf16 ? chunk_states_bf16 : at<float>(workspace, plan.hbf)) : nullptr;
  if (plan.bf16)
    SSD_LAUNCH(ssd::launch_chunk_state_fwd_bf16(d, x, B, dt, A_log, init_state, states, final_state, hbf, st),
               "chunk_state_fwd");
  else
    SSD_LAUNCH(ssd::launch_chunk_state_fwd(d, act, x, B, dt, A_log, init_state, states, final_state, nullptr,
                                           at<float>(workspace, plan.send), st),
               "chunk_state_fwd");
  if (plan.bf16)
    SSD_LAUNCH(ssd::launch_out_fwd_bf16(d, choose_nsplit(d, kFwdTarget, true), x, B, C, dt, A_log, D, hbf, y, st),
               "chunk_out_fwd");
  else {
    const GeneralShape sh = general_fwd_shape(d);
    SSD_LAUNCH(ssd::launch_chunk_out_fwd(d, act, sh.nsplit, sh.paired, x, B, C, dt, A_log, D, states, y, st),
               "chunk_out_fwd");
  }
  return ok();
}

}  // extern "C"

namespace {

// The scratch of ssd_bwd_noalloc: one array per GPU, located per device with
// hipGetSymbolAddress (its name is a host-side stand-in for the device
// address and is never passed to a kernel).
__device__ __align__(256) char scratch[SSD_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // indexed by device ordinal

// The device address of this device's scratch (taken once per device, with
// that device current).
int noalloc_scratch(hipStream_t st, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "ssd_bwd_noalloc: hipGetDevice failed: %s", hipGetErrorString(e));
  if (st) {
    int sdev = -1;
    e = hipStreamGetDevice(st, &sdev);
    if (e != hipSuccess)
      return fail(SSD_ERR_HIP, "ssd_bwd_noalloc: hipStreamGetDevice failed: %s", hipGetErrorString(e));
    if (sdev != dev)
      return fail(SSD_ERR_INVALID_ARG, "ssd_bwd_noalloc: the stream belongs to device %d, the current device is %d",
                  sdev, dev);
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (static_cast<int>(g_scratch_ptr.size()) <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SSD_ERR_HIP, "ssd_bwd_noalloc: hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SSD_OK;
}

int bwd_impl(const char* who, const ssd_problem* prob, const void* x, const void* dt, const float* A_log,
             const void* B, const void* C, const float* D, const float* init_state, const float* chunk_states,
             const void* chunk_states_bf16, const void* dy, const float* d_final_state, float* dx, float* ddt, float* dA_log, float* dB, float* dC,
             float* dD, float* d_init_state, void* workspace, size_t workspace_bytes, bool noalloc, void* stream) {
  ssd::Dims d;
  int rc = check_problem(prob, &d);
  if (rc != SSD_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const ssd::DType act = static_cast<ssd::DType>(prob->act_dtype);
  const ssd::DType dyt = static_cast<ssd::DType>(prob->dy_dtype);
  if (!A_log || !D || !dA_log || !dD) return fail(SSD_ERR_INVALID_ARG, "%s: A_log, D, dA_log and dD are required", who);
  const bool empty = d.b == 0 || d.T == 0;
  if (!empty && (!x || !dt || !B || !C || !dy || !dx || !ddt || !dB || !dC))
    return fail(SSD_ERR_INVALID_ARG, "%s: x, dt, B, C, dy, dx, ddt, dB and dC are required", who);
  const void* ptrs[] = {x,  dt,  A_log,  B,  C,  D,  init_state,   chunk_states, chunk_states_bf16, dy, d_final_state,
                        dx, ddt, dA_log, dB, dC, dD, d_init_state};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(SSD_ERR_ALIGN, "%s: a tensor pointer is not 16-byte aligned", who);
  if (empty) {
    SSD_LAUNCH(ssd::launch_fill(dA_log, d.H, 0.f, st), "fill");
    SSD_LAUNCH(ssd::launch_fill(dD, d.H, 0.f, st), "fill");
    if (d_init_state) {
      const int64_t n = static_cast<int64_t>(d.b) * d.H * d.P * d.N;
      // no steps: the final state is the initial one
      if (d_final_state)
        SSD_LAUNCH(ssd::launch_copy(d_init_state, d_final_state, n, st), "copy");
      else
        SSD_LAUNCH(ssd::launch_fill(d_init_state, n, 0.f, st), "fill");
    }
    return ok();
  }
  if (chunk_states_bf16 && !use_bf16_kernels(d, prob->act_dtype, prob->dy_dtype))
    return fail(SSD_ERR_INVALID_ARG,
                "%s: chunk_states_bf16 needs a problem the bf16 kernels run (bf16 activations and dy, headdim and "
                "dstate multiples of 8)",
                who);
  const BwdPlan plan = plan_bwd(d, chunk_states != nullptr, use_bf16_kernels(d, prob->act_dtype, prob->dy_dtype));
  if (noalloc) {
    if (plan.total > SSD_NOALLOC_SCRATCH_BYTES)
      return fail(SSD_ERR_WORKSPACE,
                  "%s: the problem needs %zu bytes of scratch, more than the %zu of the library's static scratch "
                  "(use ssd_bwd with a workspace%s)",
                  who, plan.total, static_cast<size_t>(SSD_NOALLOC_SCRATCH_BYTES),
                  chunk_states ? "" : ", or pass the saved chunk states");
    rc = noalloc_scratch(static_cast<hipStream_t>(stream), &workspace);
    if (rc != SSD_OK) return rc;
    workspace_bytes = SSD_NOALLOC_SCRATCH_BYTES;
  }
  if (!workspace) return fail(SSD_ERR_WORKSPACE, "%s: workspace is null (%zu bytes needed)", who, plan.total);
  if (workspace_bytes < plan.total)
    return fail(SSD_ERR_WORKSPACE, "%s: workspace of %zu bytes is smaller than the %zu needed", who, workspace_bytes,
                plan.total);
  if (!aligned16(workspace)) return fail(SSD_ERR_ALIGN, "%s: workspace is not 16-byte aligned", who);

  ssd::BwdScratch s;
  s.rowM = at<float>(workspace, plan.rowM);
  s.colE = at<float>(workspace, plan.colE);
  s.diagE = at<float>(workspace, plan.diagE);
  s.Rp = at<float>(workspace, plan.Rp);
  s.dsoff = at<float>(workspace, plan.dsoff);
  s.gh_part = at<float>(workspace, plan.gh);
  s.dA_part = at<float>(workspace, plan.dA);
  s.dD_part = at<float>(workspace, plan.dD);
  s.done = at<unsigned>(workspace, plan.done);
  s.wstrips = plan.fused ? at<uint16_t>(workspace, plan.wst) : nullptr;
  s.dB_part = plan.nsplit > 1 ? at<float>(workspace, plan.dB) : nullptr;
  s.dC_part = plan.nsplit > 1 ? at<float>(workspace, plan.dC) : nullptr;
  s.row_slots = plan.fused ? d.nb() : 0;
  s.slot_elems = static_cast<int64_t>(d.b) * d.H * d.T;
  void* gamma = at<float>(workspace, plan.gamma);
  void* hbf = plan.bf16 ? at<float>(workspace, plan.hbf) : nullptr;

  if (plan.fused) {
    // The fused kernel reads H_c in bf16 and forms <Gamma_{c+1}, H_c> itself,
    // so the reverse pass needs H_c only to make the bf16 copy: not at all
    // with the saved bf16 history, from the f32 history otherwise, and
    // without a history the forward chunk-state kernel recomputes the bf16
    // copy alone.
    const float* hstates = nullptr;
    void* hbf_out = nullptr;
    if (chunk_states_bf16) {
      hbf = const_cast<void*>(chunk_states_bf16);
    } else if (chunk_states) {
      hstates = chunk_states;
      hbf_out = hbf;
    } else {
      SSD_LAUNCH(ssd::launch_chunk_state_fwd_bf16(d, x, B, dt, A_log, init_state, nullptr, nullptr, hbf, st),
                 "chunk_state_fwd (recompute)");
    }
    SSD_LAUNCH(ssd::launch_chunk_state_bwd_bf16(d, dy, C, dt, A_log, d_final_state, hstates, gamma, d_init_state,
                                                nullptr, hbf_out, s.done, st),
               "chunk_state_bwd");
    // the fused kernel also does the dt kernel's work (ddt, dA_log, dD)
    SSD_LAUNCH(ssd::launch_bwd_fused_bf16(d, plan.nsplit, x, B, C, dt, dy, A_log, D, gamma, hbf, dx,
                                          plan.nsplit > 1 ? s.dB_part : dB, plan.nsplit > 1 ? s.dC_part : dC, ddt,
                                          dA_log, dD, s, st),
               "chunk_bwd_fused");
    if (plan.nsplit > 1) SSD_LAUNCH(ssd::launch_bwd_split_sum(d, plan.nsplit, dB, dC, s, st), "bwd_split_sum");
    return ok();
  }

  // the split bf16 form and the general family: the f32 states (the bf16
  // history, if given, is not used)
  const float* states = chunk_states;
  if (!states) {
    float* rec = at<float>(workspace, plan.states);
    // the same kernel as ssd_fwd picks, so recomputed states match saved ones bitwise
    if (use_bf16_kernels(d, prob->act_dtype, prob->act_dtype))
      SSD_LAUNCH(ssd::launch_chunk_state_fwd_bf16(d, x, B, dt, A_log, init_state, rec, nullptr, nullptr, st),
                 "chunk_state_fwd (recompute)");
    else
      SSD_LAUNCH(ssd::launch_chunk_state_fwd(d, act, x, B, dt, A_log, init_state, rec, nullptr, nullptr,
                                             at<float>(workspace, plan.send), st),
                 "chunk_state_fwd (recompute)");
    states = rec;
  }
  if (plan.bf16)
    SSD_LAUNCH(ssd::launch_chunk_state_bwd_bf16(d, dy, C, dt, A_log, d_final_state, states, gamma, d_init_state,
                                                s.gh_part, hbf, nullptr, st),
               "chunk_state_bwd");
  else
    SSD_LAUNCH(
        ssd::launch_chunk_state_bwd(d, act, dyt, dy, C, dt, A_log, d_final_state, states, gamma, d_init_state,
                                    s.gh_part, nullptr, at<float>(workspace, plan.send), st),
        "chunk_state_bwd");
  if (plan.bf16) {
    SSD_LAUNCH(ssd::launch_bwd_col_bf16(d, plan.nsplit, x, B, C, dt, dy, A_log, D, gamma, dx,
                                        plan.nsplit > 1 ? s.dB_part : dB, s, st),
               "chunk_bwd_col");
    SSD_LAUNCH(ssd::launch_bwd_row_bf16(d, plan.nsplit, x, B, C, dt, dy, A_log, hbf,
                                        plan.nsplit > 1 ? s.dC_part : dC, s, st),
               "chunk_bwd_row");
  } else {
    SSD_LAUNCH(ssd::launch_chunk_bwd_col(d, act, dyt, plan.nsplit, plan.paired, x, B, C, dt, dy, A_log, D, gamma, dx,
                                         plan.nsplit > 1 ? s.dB_part : dB, s, st),
               "chunk_bwd_col");
    SSD_LAUNCH(ssd::launch_chunk_bwd_row(d, act, dyt, plan.nsplit, plan.paired, x, B, C, dt, dy, A_log, states,
                                         plan.nsplit > 1 ? s.dC_part : dC, s, st),
               "chunk_bwd_row");
  }
  SSD_LAUNCH(ssd::launch_bwd_dt(d, act, dt, A_log, ddt, dA_log, dD, s, st), "bwd_dt");
  if (plan.nsplit > 1) SSD_LAUNCH(ssd::launch_bwd_split_sum(d, plan.nsplit, dB, dC, s, st), "bwd_split_sum");
  return ok();
}

}  // namespace

extern "C" {

int ssd_bwd(const ssd_problem* prob, const void* x, const void* dt, const float* A_log, const void* B,
            const void* C, const float* D, const float* init_state, const float* chunk_states, const void* dy,
            const float* d_final_state, float* dx, float* ddt, float* dA_log, float* dB, float* dC, float* dD,
            float* d_init_state, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl("ssd_bwd", prob, x, dt, A_log, B, C, D, init_state, chunk_states, nullptr, dy, d_final_state, dx,
                  ddt, dA_log, dB, dC, dD, d_init_state, workspace, workspace_bytes, false, stream);
}

int ssd_bwd_ex(const ssd_problem* prob, const void* x, const void* dt, const float* A_log, const void* B,
               const void* C, const float* D, const float* init_state, const float* chunk_states,
               const void* chunk_states_bf16, const void* dy, const float* d_final_state, float* dx, float* ddt,
               float* dA_log, float* dB, float* dC, float* dD, float* d_init_state, void* workspace,
               size_t workspace_bytes, void* stream) {
  return bwd_impl("ssd_bwd_ex", prob, x, dt, A_log, B, C, D, init_state, chunk_states, chunk_states_bf16, dy,
                  d_final_state, dx, ddt, dA_log, dB, dC, dD, d_init_state, workspace, workspace_bytes, false, stream);
}

int ssd_bwd_noalloc(const ssd_problem* prob, const void* x, const void* dt, const float* A_log, const void* B,
                    const void* C, const float* D, const float* init_state, const float* chunk_states,
                    const void* dy, const float* d_final_state, float* dx, float* ddt, float* dA_log, float* dB,
                    float* dC, float* dD, float* d_init_state, void* stream) {
  g_prof_suppress = true;
  const int rc = bwd_impl("ssd_bwd_noalloc", prob, x, dt, A_log, B, C, D, init_state, chunk_states, nullptr, dy,
                          d_final_state, dx, ddt, dA_log, dB, dC, dD, d_init_state, nullptr, 0, true, stream);
  g_prof_suppress = false;
  return rc;
}

// ------------------------------------------------------------------ shell

static int check_conv(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t ngroups, int64_t dstate,
                      int64_t d_conv, int32_t dtype) {
  if (!valid_dtype(dtype)) return fail(SSD_ERR_DTYPE, "conv1d: dtype %d is not SSD_F32 or SSD_BF16", dtype);
  if (batch < 0 || seqlen < 0 || d_inner <= 0 || ngroups <= 0 || dstate <= 0 || d_conv <= 0)
    return fail(SSD_ERR_INVALID_ARG, "conv1d: sizes must be positive (batch, seqlen >= 0)");
  if (d_conv > ssd::conv_max_k()) return fail(SSD_ERR_SHAPE, "conv1d: d_conv %lld exceeds %d", (long long)d_conv, ssd::conv_max_k());
  if (batch > 65535 || seqlen > (int64_t(1) << 30) || d_inner + 2 * ngroups * dstate > (int64_t(1) << 24))
    return fail(SSD_ERR_SHAPE, "conv1d: problem too large");
  return SSD_OK;
}

size_t mamba2_conv1d_silu_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t ngroups,
                                              int64_t dstate, int64_t d_conv) {
  if (check_conv(batch, seqlen, d_inner, ngroups, dstate, d_conv, SSD_F32) != SSD_OK) return 0;
  if (batch == 0 || seqlen == 0) return 0;
  const int64_t cd = d_inner + 2 * ngroups * dstate;
  return align_up(sizeof(float) * static_cast<size_t>(batch) * ssd::conv_nruns(static_cast<int>(seqlen)) * cd *
                  (d_conv + 1));
}

int mamba2_conv1d_silu_fwd(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t ngroups, int64_t dstate,
                           int64_t d_conv, int32_t dtype, const void* xbc, const float* w, const float* bias,
                           void* x_out, void* B_out, void* C_out, void* stream) {
  int rc = check_conv(batch, seqlen, d_inner, ngroups, dstate, d_conv, dtype);
  if (rc != SSD_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (batch == 0 || seqlen == 0) return ok();
  if (!xbc || !w || !x_out || !B_out || !C_out)
    return fail(SSD_ERR_INVALID_ARG, "conv1d_silu_fwd: xbc, w, x_out, B_out and C_out are required");
  const void* ptrs[] = {xbc, w, bias, x_out, B_out, C_out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(SSD_ERR_ALIGN, "conv1d_silu_fwd: a tensor pointer is not 16-byte aligned");
  SSD_LAUNCH(ssd::launch_conv_fwd(static_cast<int>(batch), static_cast<int>(seqlen), static_cast<int>(d_inner),
                                  static_cast<int>(ngroups * dstate), static_cast<int>(d_conv),
                                  static_cast<ssd::DType>(dtype), xbc, w, bias, x_out, B_out, C_out, st),
             "conv1d_silu_fwd");
  return ok();
}

int mamba2_conv1d_silu_bwd(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t ngroups, int64_t dstate,
                           int64_t d_conv, int32_t dtype, const void* xbc, const float* w, const float* bias,
                           const float* dx, const float* dB, const float* dC, int32_t dxbc_dtype, void* dxbc,
                           int64_t dxbc_ld, float* dw, float* dbias, void* workspace, size_t workspace_bytes,
                           void* stream) {
  int rc = check_conv(batch, seqlen, d_inner, ngroups, dstate, d_conv, dtype);
  if (rc != SSD_OK) return rc;
  if (!valid_dtype(dxbc_dtype))
    return fail(SSD_ERR_DTYPE, "conv1d_silu_bwd: dxbc_dtype %d is not SSD_F32 or SSD_BF16", dxbc_dtype);
  if (!dw || !dbias) return fail(SSD_ERR_INVALID_ARG, "conv1d_silu_bwd: dw and dbias are required");
  const int64_t cd = d_inner + 2 * ngroups * dstate;
  if (dxbc_ld == 0) dxbc_ld = cd;
  // a wider row keeps its elements 16 bytes (f32) or 8 bytes (bf16) aligned
  // in groups of four, as the vector kernel stores them
  if (dxbc_ld < cd || (dxbc_ld != cd && dxbc_ld % 4 != 0))
    return fail(SSD_ERR_INVALID_ARG, "conv1d_silu_bwd: dxbc_ld %lld must be 0, %lld, or a multiple of 4 above it",
                (long long)dxbc_ld, (long long)cd);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (batch == 0 || seqlen == 0) {
    SSD_LAUNCH(ssd::launch_fill(dw, cd * d_conv, 0.f, st), "fill");
    SSD_LAUNCH(ssd::launch_fill(dbias, cd, 0.f, st), "fill");
    return ok();
  }
  if (!xbc || !w || !dx || !dB || !dC || !dxbc)
    return fail(SSD_ERR_INVALID_ARG, "conv1d_silu_bwd: xbc, w, dx, dB, dC and dxbc are required");
  const void* ptrs[] = {xbc, w, bias, dx, dB, dC, dxbc, dw, dbias, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(SSD_ERR_ALIGN, "conv1d_silu_bwd: a pointer is not 16-byte aligned");
  const size_t need = mamba2_conv1d_silu_bwd_workspace_bytes(batch, seqlen, d_inner, ngroups, dstate, d_conv);
  if (!workspace || workspace_bytes < need)
    return fail(SSD_ERR_WORKSPACE, "conv1d_silu_bwd: workspace of %zu bytes is smaller than the %zu needed",
                workspace ? workspace_bytes : 0, need);
  SSD_LAUNCH(ssd::launch_conv_bwd(static_cast<int>(batch), static_cast<int>(seqlen), static_cast<int>(d_inner),
                                  static_cast<int>(ngroups * dstate), static_cast<int>(d_conv),
                                  static_cast<ssd::DType>(dtype), xbc, w, bias, dx, dB, dC, dxbc,
                                  static_cast<ssd::DType>(dxbc_dtype), dxbc_ld, dw, dbias,
                                  static_cast<float*>(workspace), st),
             "conv1d_silu_bwd");
  return ok();
}

static int check_rms(int64_t rows, int64_t width, int32_t dtype) {
  if (!valid_dtype(dtype)) return fail(SSD_ERR_DTYPE, "rmsnorm_gated: dtype %d is not SSD_F32 or SSD_BF16", dtype);
  if (rows < 0 || width <= 0) return fail(SSD_ERR_INVALID_ARG, "rmsnorm_gated: rows >= 0 and width > 0 required");
  if (width > ssd::rms_max_width())
    return fail(SSD_ERR_SHAPE, "rmsnorm_gated: width %lld exceeds %d", (long long)width, ssd::rms_max_width());
  if (rows > (int64_t(1) << 31) - 1) return fail(SSD_ERR_SHAPE, "rmsnorm_gated: too many rows");
  return SSD_OK;
}

size_t mamba2_rmsnorm_gated_bwd_workspace_bytes(int64_t rows, int64_t width) {
  if (check_rms(rows, width, SSD_F32) != SSD_OK || rows == 0) return 0;
  return align_up(sizeof(float) * static_cast<size_t>(ssd::rms_nparts(rows)) * width);
}

int mamba2_rmsnorm_gated_fwd(int64_t rows, int64_t width, float eps, int32_t dtype, const void* y, const void* z,
                             const float* w, void* out, float* inv_rms, void* stream) {
  int rc = check_rms(rows, width, dtype);
  if (rc != SSD_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (rows == 0) return ok();
  if (!y || !z || !w || !out || !inv_rms)
    return fail(SSD_ERR_INVALID_ARG, "rmsnorm_gated_fwd: y, z, w, out and inv_rms are required");
  if (!(eps >= 0.f)) return fail(SSD_ERR_INVALID_ARG, "rmsnorm_gated_fwd: eps must be >= 0");
  const void* ptrs[] = {y, z, w, out, inv_rms};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(SSD_ERR_ALIGN, "rmsnorm_gated_fwd: a tensor pointer is not 16-byte aligned");
  SSD_LAUNCH(ssd::launch_rms_fwd(rows, static_cast<int>(width), eps, static_cast<ssd::DType>(dtype), y, z, w, out,
                                 inv_rms, st),
             "rmsnorm_gated_fwd");
  return ok();
}

int mamba2_rmsnorm_gated_bwd(int64_t rows, int64_t width, int32_t dtype, int32_t g_dtype, int32_t dy_dtype,
                             int32_t dz_dtype, const void* y, const void* z, const float* w, const float* inv_rms,
                             const void* g, void* dy, void* dz, int64_t dz_ld, float* dw, void* workspace,
                             size_t workspace_bytes, void* stream) {
  int rc = check_rms(rows, width, dtype);
  if (rc != SSD_OK) return rc;
  if (!valid_dtype(g_dtype)) return fail(SSD_ERR_DTYPE, "rmsnorm_gated_bwd: g_dtype %d is not SSD_F32 or SSD_BF16", g_dtype);
  if (!valid_dtype(dy_dtype))
    return fail(SSD_ERR_DTYPE, "rmsnorm_gated_bwd: dy_dtype %d is not SSD_F32 or SSD_BF16", dy_dtype);
  if (!valid_dtype(dz_dtype))
    return fail(SSD_ERR_DTYPE, "rmsnorm_gated_bwd: dz_dtype %d is not SSD_F32 or SSD_BF16", dz_dtype);
  if (dz_ld == 0) dz_ld = width;
  // a wider row keeps the 16-byte groups of eight that the vector kernel stores aligned
  if (dz_ld < width || (dz_ld != width && dz_ld % 8 != 0))
    return fail(SSD_ERR_INVALID_ARG, "rmsnorm_gated_bwd: dz_ld %lld must be 0, %lld, or a multiple of 8 above it",
                (long long)dz_ld, (long long)width);
  if (!dw) return fail(SSD_ERR_INVALID_ARG, "rmsnorm_gated_bwd: dw is required");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (rows == 0) {
    SSD_LAUNCH(ssd::launch_fill(dw, width, 0.f, st), "fill");
    return ok();
  }
  if (!y || !z || !w || !inv_rms || !g || !dy || !dz)
    return fail(SSD_ERR_INVALID_ARG, "rmsnorm_gated_bwd: y, z, w, inv_rms, g, dy and dz are required");
  const void* ptrs[] = {y, z, w, inv_rms, g, dy, dz, dw, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(SSD_ERR_ALIGN, "rmsnorm_gated_bwd: a pointer is not 16-byte aligned");
  const size_t need = mamba2_rmsnorm_gated_bwd_workspace_bytes(rows, width);
  if (!workspace || workspace_bytes < need)
    return fail(SSD_ERR_WORKSPACE, "rmsnorm_gated_bwd: workspace of %zu bytes is smaller than the %zu needed",
                workspace ? workspace_bytes : 0, need);
  SSD_LAUNCH(ssd::launch_rms_bwd(rows, static_cast<int>(width), static_cast<ssd::DType>(dtype),
                                 static_cast<ssd::DType>(g_dtype), static_cast<ssd::DType>(dy_dtype), y, z, w,
                                 inv_rms, g, dy, dz, static_cast<ssd::DType>(dz_dtype), dz_ld, dw,
                                 static_cast<float*>(workspace), st),
             "rmsnorm_gated_bwd");
  return ok();
}

// ------------------------------------------------------------ dt activation

static int check_dt(int64_t rows, int64_t nheads, int32_t dtype) {
  if (!valid_dtype(dtype)) return fail(SSD_ERR_DTYPE, "dt_softplus: dtype %d is not SSD_F32 or SSD_BF16", dtype);
  if (rows < 0 || nheads <= 0) return fail(SSD_ERR_INVALID_ARG, "dt_softplus: rows >= 0 and nheads > 0 required");
  if (nheads > (int64_t(1) << 20) || rows > (int64_t(1) << 40) / nheads)
    return fail(SSD_ERR_SHAPE, "dt_softplus: rows x nheads is too large");
  return SSD_OK;
}

int ssd_dt_softplus_fwd(int64_t rows, int64_t nheads, int32_t dtype, const void* dt_raw, const float* dt_bias,
                        void* dt, void* stream) {
  int rc = check_dt(rows, nheads, dtype);
  if (rc != SSD_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (rows == 0) return ok();
  if (!dt_raw || !dt_bias || !dt)
    return fail(SSD_ERR_INVALID_ARG, "dt_softplus_fwd: dt_raw, dt_bias and dt are required");
  const void* ptrs[] = {dt_raw, dt_bias, dt};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(SSD_ERR_ALIGN, "dt_softplus_fwd: a tensor pointer is not 16-byte aligned");
  SSD_LAUNCH(ssd::launch_dt_softplus_fwd(rows, static_cast<int>(nheads), static_cast<ssd::DType>(dtype), dt_raw,
                                         dt_bias, dt, st),
             "dt_softplus_fwd");
  return ok();
}

size_t ssd_dt_softplus_bwd_workspace_bytes(int64_t rows, int64_t nheads) {
  if (check_dt(rows, nheads, SSD_F32) != SSD_OK || rows == 0) return 0;
  return align_up(sizeof(float) * static_cast<size_t>(ssd::dt_nparts(rows)) * nheads);
}

int ssd_dt_softplus_bwd(int64_t rows, int64_t nheads, int32_t dtype, const void* dt_raw, const float* dt_bias,
                        const float* ddt, int32_t ddt_raw_dtype, void* ddt_raw, int64_t ddt_raw_ld,
                        float* d_dt_bias, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_dt(rows, nheads, dtype);
  if (rc != SSD_OK) return rc;
  if (!valid_dtype(ddt_raw_dtype))
    return fail(SSD_ERR_DTYPE, "dt_softplus_bwd: ddt_raw_dtype %d is not SSD_F32 or SSD_BF16", ddt_raw_dtype);
  if (ddt_raw_ld == 0) ddt_raw_ld = nheads;
  if (ddt_raw_ld < nheads)
    return fail(SSD_ERR_INVALID_ARG, "dt_softplus_bwd: ddt_raw_ld %lld is below nheads %lld",
                (long long)ddt_raw_ld, (long long)nheads);
  if (!d_dt_bias) return fail(SSD_ERR_INVALID_ARG, "dt_softplus_bwd: d_dt_bias is required");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (rows == 0) {
    SSD_LAUNCH(ssd::launch_fill(d_dt_bias, nheads, 0.f, st), "fill");
    return ok();
  }
  if (!dt_raw || !dt_bias || !ddt || !ddt_raw)
    return fail(SSD_ERR_INVALID_ARG, "dt_softplus_bwd: dt_raw, dt_bias, ddt and ddt_raw are required");
  const void* ptrs[] = {dt_raw, dt_bias, ddt, ddt_raw, d_dt_bias, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(SSD_ERR_ALIGN, "dt_softplus_bwd: a pointer is not 16-byte aligned");
  const size_t need = ssd_dt_softplus_bwd_workspace_bytes(rows, nheads);
  if (!workspace || workspace_bytes < need)
    return fail(SSD_ERR_WORKSPACE, "dt_softplus_bwd: workspace of %zu bytes is smaller than the %zu needed",
                workspace ? workspace_bytes : 0, need);
  SSD_LAUNCH(ssd::launch_dt_softplus_bwd(rows, static_cast<int>(nheads), static_cast<ssd::DType>(dtype), dt_raw,
                                         dt_bias, ddt, ddt_raw, static_cast<ssd::DType>(ddt_raw_dtype), ddt_raw_ld,
                                         d_dt_bias, static_cast<float*>(workspace), st),
             "dt_softplus_bwd");
  return ok();
}

// ------------------------------------------------------------ projections

int ssd_gemm(int32_t trans_a, int32_t trans_b, int64_t m, int64_t n, int64_t k, float alpha, const void* A,
             int64_t lda, const void* B, int64_t ldb, float beta, void* C, int32_t c_dtype, int64_t ldc,
             void* stream) {
  if (!valid_dtype(c_dtype)) return fail(SSD_ERR_DTYPE, "gemm: c_dtype %d is not SSD_F32 or SSD_BF16", c_dtype);
  if (m < 0 || n < 0 || k < 0) return fail(SSD_ERR_INVALID_ARG, "gemm: m, n, k must be >= 0");
  if (m == 0 || n == 0) return ok();
  if (!C || (k > 0 && (!A || !B))) return fail(SSD_ERR_INVALID_ARG, "gemm: A, B and C are required");
  // row strides: op(A) rows of k (A stored [m,k]) or A stored [k,m]; likewise B
  if (lda < (trans_a ? m : k) || ldb < (trans_b ? k : n) || ldc < n || lda < 1 || ldb < 1)
    return fail(SSD_ERR_SHAPE, "gemm: a row stride is shorter than its row");
  const void* ptrs[] = {A, B, C};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(SSD_ERR_ALIGN, "gemm: a matrix pointer is not 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t p_ = prof_begin(st, "gemm");
  const ssd::GemmStatus gs = ssd::gemm_bf16(trans_a != 0, trans_b != 0, m, n, k, alpha, A, lda, B, ldb, beta, C,
                                            c_dtype == SSD_BF16, ldc, st);
  if (gs == ssd::GemmStatus::kHip) return fail(SSD_ERR_HIP, "gemm: no current HIP device");
  if (gs == ssd::GemmStatus::kBlas) return fail(SSD_ERR_HIP, "gemm: rocBLAS gemm_ex failed");
  prof_end(p_, "gemm", st);
  return ok();
}

int ssd_cast_f32_to_bf16(int64_t n, const float* src, void* dst, void* stream) {
  if (n < 0) return fail(SSD_ERR_INVALID_ARG, "cast: n must be >= 0");
  if (n == 0) return ok();
  if (!src || !dst) return fail(SSD_ERR_INVALID_ARG, "cast: src and dst are required");
  if (!aligned16(src) || !aligned16(dst)) return fail(SSD_ERR_ALIGN, "cast: a pointer is not 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  SSD_LAUNCH(ssd::launch_cast_bf16(n, src, dst, st), "cast_bf16");
  return ok();
}

}  // extern "C"
