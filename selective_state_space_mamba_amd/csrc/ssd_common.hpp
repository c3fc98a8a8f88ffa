// Device building blocks shared by the SSD kernels (gfx950, wave64).
//
// MFMA tiles are 16x16 (v_mfma_f32_16x16x4_f32 for f32 operands,
// v_mfma_f32_16x16x32_bf16 for bf16 operands), both accumulating in f32.
// Lane l of a wave holds r = l % 16, q = l / 16; operand fragments are
//   f32 : A[r][k0+q],          B[k0+q][r]
//   bf16: A[r][k0+8q .. +7],   B[k0+8q .. +7][r]
// and the 16x16 f32 result element i (0..3) of lane l is C[4q+i][r].
//
// Operands are staged in LDS.  A "view" of an LDS matrix gives the element
// (row, k) at p[row*sr + k*sk]; when sk == 1 (k contiguous) a bf16 fragment is
// one 16-byte LDS read, otherwise eight 2-byte reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int WAVE = 64;
constexpr int NTHREADS = 256;  // 4 waves per workgroup
constexpr int BQ = 64;         // rows per block of a chunk
constexpr int PMAX = 64;       // largest headdim the kernels take
constexpr int NMAX = 128;      // largest d_state the kernels take
constexpr int QMAX = 256;      // largest chunk the kernels take
constexpr int NBMAX = QMAX / BQ;

// ---------------------------------------------------------------- scalars

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// f32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float load_f(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_f(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }

__device__ __forceinline__ void store_f(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_f(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16_bits(v); }

// ------------------------------------------------------------- MFMA types

template <bool BF> struct Op;
template <> struct Op<false> {
  typedef float T;  // LDS element
  typedef float V;  // fragment
  static constexpr int KS = 4;
  static __device__ __forceinline__ T cvt(float v) { return v; }
  static __device__ __forceinline__ float back(T v) { return v; }
};
template <> struct Op<true> {
  typedef uint16_t T;
  typedef bf16x8 V;
  static constexpr int KS = 32;
  static __device__ __forceinline__ T cvt(float v) { return f32_to_bf16_bits(v); }
  static __device__ __forceinline__ float back(T v) { return bf16_bits_to_f32(v); }
};

__device__ __forceinline__ f4 mfma(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma(bf16x8 a, bf16x8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A per-lane index the compiler must take as computed here: comparisons
// derived from it stay in the branch that uses them instead of being hoisted
// out of the loops as lane masks (which then spill to VGPR lanes).
__device__ __forceinline__ int opaque_index(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }
// Uniform across the wave; readfirstlane lets the compiler keep it, and the
// LDS and tile addresses derived from it, in scalar registers.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE); }

// Fragment of rows r0..r0+15 and k-slice starting at k0 of an LDS view.
template <bool BF, bool KC>
__device__ __forceinline__ typename Op<BF>::V fetch(const typename Op<BF>::T* p, int sr, int sk,
                                                    int r0, int k0) {
  const int l = lane_id(), r = l & 15, q = l >> 4;
  if constexpr (!BF) {
    return p[(r0 + r) * sr + (k0 + q) * sk];
  } else if constexpr (KC) {
    return *reinterpret_cast<const bf16x8*>(p + (r0 + r) * sr + k0 + 8 * q);
  } else {
    bf16x8 v;
    const uint16_t* b = p + (r0 + r) * sr + (k0 + 8 * q) * sk;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __builtin_bit_cast(__bf16, b[e * sk]);
    return v;
  }
}

// acc[t] (16 x 16, columns 16t..16t+15) += A(16 x K) * B(K x 16*NT), where
// A is the view (row = output row, k) and B the view (row = output column, k).
// K must be a multiple of Op<BF>::KS; the LDS operands are zero beyond the
// logical extent.
// V4 (f32 only): the 16-byte reads below; false keeps one 4-byte read per
// k-step (fewer registers held across the reads).
template <bool BF, bool AKC, bool BKC, int NT, bool V4 = true>
__device__ __forceinline__ void wave_gemm(f4 (&acc)[NT], const typename Op<BF>::T* A, int asr,
                                          int ask, const typename Op<BF>::T* B, int bsr, int bsk,
                                          int K) {
  typedef typename Op<BF>::V V;
  constexpr int KS = Op<BF>::KS;
  if (K <= 0) return;
  if constexpr (!BF) {
    // f32: K = 4 per MFMA, one element per lane.  Lane (r, q) of MFMA u of a
    // group of four takes k = k0 + 4q + u (both operands alike, so the four
    // MFMAs still sum over k0 .. k0 + 15 exactly once): a k-contiguous
    // operand then comes as one 16-byte read of four consecutive k per lane
    // instead of four 4-byte reads.  The reads of NG groups (two for up to
    // four output tiles, else one: the same registers as eight or four
    // k-steps of single reads) are issued ahead of their MFMAs.
    constexpr int NG = NT <= 4 ? 2 : 1;
    int k0 = 0;
    for (; V4 && k0 + 16 * NG <= K; k0 += 16 * NG) {
      float a[NG][4], b[NG][NT][4];
      const int l = lane_id(), r = l & 15, q = l >> 4;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int kg = k0 + 16 * g + 4 * q;
        if constexpr (AKC) {
          const float4 v = *reinterpret_cast<const float4*>(A + r * asr + kg);
          a[g][0] = v.x, a[g][1] = v.y, a[g][2] = v.z, a[g][3] = v.w;
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) a[g][u] = A[r * asr + (kg + u) * ask];
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if constexpr (BKC) {
            const float4 v = *reinterpret_cast<const float4*>(B + (16 * t + r) * bsr + kg);
            b[g][t][0] = v.x, b[g][t][1] = v.y, b[g][t][2] = v.z, b[g][t][3] = v.w;
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) b[g][t][u] = B[(16 * t + r) * bsr + (kg + u) * bsk];
          }
        }
      }
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t] = mfma(a[g][u], b[g][t][u], acc[t]);
    }
    constexpr int KU = NT <= 4 ? 8 : 4;
    for (; k0 + KU * KS <= K; k0 += KU * KS) {
      float a[KU], b[KU][NT];
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        a[u] = fetch<false, AKC>(A, asr, ask, 0, k0 + u * KS);
#pragma unroll
        for (int t = 0; t < NT; ++t) b[u][t] = fetch<false, BKC>(B, bsr, bsk, 16 * t, k0 + u * KS);
      }
#pragma unroll
      for (int u = 0; u < KU; ++u)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = mfma(a[u], b[u][t], acc[t]);
    }
    for (; k0 < K; k0 += KS) {
      const float a = fetch<false, AKC>(A, asr, ask, 0, k0);
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = mfma(a, fetch<false, BKC>(B, bsr, bsk, 16 * t, k0), acc[t]);
    }
    return;
  }
  // the next k-step's A fragment is read from LDS while the current MFMAs run
  V a = fetch<BF, AKC>(A, asr, ask, 0, 0);
  for (int k0 = 0; k0 < K; k0 += KS) {
    const V an = (k0 + KS < K) ? fetch<BF, AKC>(A, asr, ask, 0, k0 + KS) : a;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = mfma(a, fetch<BF, BKC>(B, bsr, bsk, 16 * t, k0), acc[t]);
    a = an;
  }
}

template <int NT>
__device__ __forceinline__ void zero(f4 (&acc)[NT]) {
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
}

__device__ __forceinline__ int round_up(int v, int m) { return (v + m - 1) / m * m; }

// Sum over the 16 lanes that share q (one output row of an MFMA tile).
__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 8);
  return v;
}

// Sum over the 4 lanes that share r (one output column across the q groups).
__device__ __forceinline__ float sum_q(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Inclusive prefix sum over the threads of the workgroup.  `tmp` holds one
// float of LDS per wave.  Every thread of the workgroup must call it.
__device__ __forceinline__ float block_inclusive_scan(float v, float* tmp) {
  const int l = lane_id(), w = wave_id();
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) {
    const float t = __shfl_up(v, o);
    if (l >= o) v += t;
  }
  if (l == WAVE - 1) tmp[w] = v;
  __syncthreads();
  float off = 0.f;
  for (int i = 0; i < w; ++i) off += tmp[i];
  __syncthreads();
  return v + off;
}

// Copy a rows x cols tile from global memory (row r at src + r*ld_src, columns
// contiguous) into LDS, converting to the operand type.  Elements with
// r >= rows_valid or c >= cols_valid are written as zero.  Transposed (TR)
// writes put element (r, c) at dst[c*ld_dst + r], else dst[r*ld_dst + c].
// Optional per-row scale.
template <typename TS, typename TD, bool TR>
__device__ __forceinline__ void stage_tile(TD* dst, int ld_dst, const TS* src, int64_t ld_src,
                                           int rows, int cols, int rows_valid, int cols_valid,
                                           const float* row_scale = nullptr) {
  for (int idx = threadIdx.x; idx < rows * cols; idx += NTHREADS) {
    const int r = idx / cols, c = idx % cols;
    float v = 0.f;
    if (r < rows_valid && c < cols_valid) {
      v = load_f(src, r * ld_src + c);
      if (row_scale) v *= row_scale[r];
    }
    TD o;
    if constexpr (sizeof(TD) == 4)
      o = v;
    else
      o = f32_to_bf16_bits(v);
    if constexpr (TR)
      dst[c * ld_dst + r] = o;
    else
      dst[r * ld_dst + c] = o;
  }
}

// ------------------------------------------------------------- staging

// Raw 16-byte global loads.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ bool vec16_ok(const void* base, int64_t ld_elems, int elem_bytes) {
  return (reinterpret_cast<uintptr_t>(base) & 15u) == 0 && ((ld_elems * elem_bytes) & 15) == 0;
}

// Eight consecutive source elements held in registers.
template <typename TS> struct Vec8;
template <> struct Vec8<uint16_t> {
  uint4 v;  // 8 bf16
  __device__ __forceinline__ float get(int e) const {
    const uint32_t w = (&v.x)[e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
  __device__ __forceinline__ void load(const uint16_t* p) { v = ld16(p); }
  __device__ __forceinline__ void load_guarded(const uint16_t* p, int n) {
    uint16_t t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = e < n ? p[e] : uint16_t(0);
    v.x = t[0] | (uint32_t(t[1]) << 16);
    v.y = t[2] | (uint32_t(t[3]) << 16);
    v.z = t[4] | (uint32_t(t[5]) << 16);
    v.w = t[6] | (uint32_t(t[7]) << 16);
  }
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
};
template <> struct Vec8<float> {
  uint4 a, b;  // 8 f32
  __device__ __forceinline__ float get(int e) const {
    return __uint_as_float(e < 4 ? (&a.x)[e] : (&b.x)[e - 4]);
  }
  __device__ __forceinline__ void load(const float* p) {
    a = ld16(p);
    b = ld16(p + 4);
  }
  __device__ __forceinline__ void load_guarded(const float* p, int n) {
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = e < n ? p[e] : 0.f;
    a = make_uint4(__float_as_uint(t[0]), __float_as_uint(t[1]), __float_as_uint(t[2]), __float_as_uint(t[3]));
    b = make_uint4(__float_as_uint(t[4]), __float_as_uint(t[5]), __float_as_uint(t[6]), __float_as_uint(t[7]));
  }
  __device__ __forceinline__ void zero() { a = b = make_uint4(0, 0, 0, 0); }
};

// Two floats -> two bf16 (round to nearest even) in one 32-bit word, low
// half first (one v_cvt_pk_bf16_f32 on gfx950).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// Store eight floats (converted to the operand type) at an LDS address that is
// 16-byte aligned for bf16 (one 16-byte write) or f32 (two).
__device__ __forceinline__ void st8(uint16_t* d, const float (&f)[8]) {
  *reinterpret_cast<uint4*>(d) =
      make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7]));
}
__device__ __forceinline__ void st8(float* d, const float (&f)[8]) {
  *reinterpret_cast<float4*>(d) = make_float4(f[0], f[1], f[2], f[3]);
  *reinterpret_cast<float4*>(d + 4) = make_float4(f[4], f[5], f[6], f[7]);
}

// 16-bit element c (0..7) of rows a and b packed as (a_c | b_c << 16).
__device__ __forceinline__ uint32_t pair16(const uint4& a, const uint4& b, int c) {
  const uint32_t wa = (&a.x)[c >> 1], wb = (&b.x)[c >> 1];
  return (c & 1) ? ((wa >> 16) | (wb & 0xFFFF0000u)) : ((wa & 0xFFFFu) | (wb << 16));
}

// Global -> LDS staging of a ROWS x COLS tile whose source rows are contiguous:
// source element (r, c) at src[r*ld + c], destination dst[r*ld_dst + c]
// (ld_dst a multiple of 8).  Elements outside rows_valid x cols_valid are zero.
// load() issues every global load of the tile into registers; store() converts
// (optionally scaling by row) and writes LDS.  Splitting the two lets a kernel
// overlap the loads of the next tile with work on the current one.
template <typename TS, int ROWS, int COLS, int NT = NTHREADS>
struct RowTile {
  static_assert(COLS % 8 == 0, "tile width must be a multiple of 8");
  static constexpr int ITEMS = ROWS * COLS / 8;
  static constexpr int PER = (ITEMS + NT - 1) / NT;
  Vec8<TS> v[PER];
  int nrows;
  __device__ __forceinline__ void load(const TS* src, int64_t ld, int rows_valid, int cols_valid) {
    nrows = rows_valid;
    const bool vec = vec16_ok(src, ld, sizeof(TS));
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int it = threadIdx.x + i * NT;
      const int r = it / (COLS / 8), c0 = (it % (COLS / 8)) * 8;
      if (it < ITEMS && r < rows_valid && c0 < cols_valid) {
        const TS* p = src + r * ld + c0;
        if (vec && c0 + 8 <= cols_valid)
          v[i].load(p);
        else
          v[i].load_guarded(p, cols_valid - c0);
      } else {
        v[i].zero();
      }
    }
  }
  template <typename TD>
  __device__ __forceinline__ void store(TD* dst, int ld_dst, const float* row_scale = nullptr) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int it = threadIdx.x + i * NT;
      if (it < ITEMS) {
        const int r = it / (COLS / 8), c0 = (it % (COLS / 8)) * 8;
        if constexpr (sizeof(TS) == 2 && sizeof(TD) == 2) {
          if (!row_scale) {
            *reinterpret_cast<uint4*>(dst + r * ld_dst + c0) = v[i].v;
            continue;
          }
        }
        const float sc = (row_scale && r < nrows) ? row_scale[r] : 1.f;
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = v[i].get(e) * sc;
        st8(dst + r * ld_dst + c0, f);
      }
    }
  }
  // Same as store() without a scale (interface shared with TransTile).
  template <typename TD>
  __device__ __forceinline__ void store_rows(TD* dst, int ld_dst) const { store(dst, ld_dst); }
};

// Global -> LDS staging with a transpose: source element (r, c) at
// src[r*ld + c] (ROWS x COLS), destination dst[c*ld_dst + r], i.e. the LDS tile
// has COLS rows of ROWS contiguous elements.  Each thread moves RB x 8 blocks
// (RB = 8 or 4 source rows) through registers: 16-bit blocks are transposed
// with byte permutes, f32 blocks converted in pairs.  Optional scale by source
// row (a time step, say).  RB = 4 halves the registers a thread holds.
template <typename TS, int ROWS, int COLS, int RB = 8, int NT = NTHREADS>
struct TransTile {
  static_assert(RB == 8 || RB == 4, "blocks of 8 or 4 rows");
  static_assert(COLS % 8 == 0 && ROWS % RB == 0, "tile sides must be multiples of the block");
  static constexpr int ITEMS = (ROWS / RB) * (COLS / 8);
  static constexpr int PER = (ITEMS + NT - 1) / NT;
  Vec8<TS> v[PER][RB];
  int nrows;
  __device__ __forceinline__ void load(const TS* src, int64_t ld, int rows_valid, int cols_valid) {
    nrows = rows_valid;
    const bool vec = vec16_ok(src, ld, sizeof(TS));
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int it = threadIdx.x + i * NT;
      const int c0 = (it % (COLS / 8)) * 8, r0 = (it / (COLS / 8)) * RB;
#pragma unroll
      for (int e = 0; e < RB; ++e) {
        const int r = r0 + e;
        if (it < ITEMS && r < rows_valid && c0 < cols_valid) {
          const TS* p = src + r * ld + c0;
          if (vec && c0 + 8 <= cols_valid)
            v[i][e].load(p);
          else
            v[i][e].load_guarded(p, cols_valid - c0);
        } else {
          v[i][e].zero();
        }
      }
    }
  }
  template <typename TD>
  __device__ __forceinline__ void store(TD* dst, int ld_dst, const float* row_scale = nullptr) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int it = threadIdx.x + i * NT;
      if (it < ITEMS) {
        const int c0 = (it % (COLS / 8)) * 8, r0 = (it / (COLS / 8)) * RB;
        if constexpr (sizeof(TS) == 2 && sizeof(TD) == 2) {
          if (!row_scale) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
              TD* d = dst + (c0 + c) * ld_dst + r0;
              if constexpr (RB == 8)
                *reinterpret_cast<uint4*>(d) =
                    make_uint4(pair16(v[i][0].v, v[i][1].v, c), pair16(v[i][2].v, v[i][3].v, c),
                               pair16(v[i][4].v, v[i][5].v, c), pair16(v[i][6].v, v[i][7].v, c));
              else
                *reinterpret_cast<uint2*>(d) = make_uint2(pair16(v[i][0].v, v[i][1].v, c), pair16(v[i][2].v, v[i][3].v, c));
            }
            continue;
          }
        }
        float sc[RB];
#pragma unroll
        for (int e = 0; e < RB; ++e) sc[e] = (row_scale && r0 + e < nrows) ? row_scale[r0 + e] : 1.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float f[RB];
#pragma unroll
          for (int e = 0; e < RB; ++e) f[e] = v[i][e].get(c) * sc[e];
          TD* d = dst + (c0 + c) * ld_dst + r0;
          if constexpr (RB == 8) {
            st8(d, f);
          } else if constexpr (sizeof(TD) == 2) {
            *reinterpret_cast<uint2*>(d) = make_uint2(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]));
          } else {
            *reinterpret_cast<float4*>(d) = make_float4(f[0], f[1], f[2], f[3]);
          }
        }
      }
    }
  }
  // The same registers written untransposed: dst[r*ld_dst + c].
  template <typename TD>
  __device__ __forceinline__ void store_rows(TD* dst, int ld_dst) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int it = threadIdx.x + i * NT;
      if (it < ITEMS) {
        const int c0 = (it % (COLS / 8)) * 8, r0 = (it / (COLS / 8)) * RB;
#pragma unroll
        for (int e = 0; e < RB; ++e) {
          if constexpr (sizeof(TS) == 2 && sizeof(TD) == 2) {
            *reinterpret_cast<uint4*>(dst + (r0 + e) * ld_dst + c0) = v[i][e].v;
          } else {
            float f[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) f[c] = v[i][e].get(c);
            st8(dst + (r0 + e) * ld_dst + c0, f);
          }
        }
      }
    }
  }
};

// Workgroups are handed to the 8 XCDs of the chip round-robin in launch order,
// so consecutive block indices land on different XCDs (different L2 caches).
// This maps the launch index to a logical index such that consecutive logical
// indices run on one XCD: workgroups that share operands then share its L2.
constexpr int NXCD = 8;
__device__ __forceinline__ int xcd_logical_block(int bid, int nblk) {
  const int per = nblk / NXCD, rem = nblk % NXCD;
  const int xcd = bid % NXCD, slot = bid / NXCD;
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;
}

}  // namespace ssd
