// Asynchronous LDS staging and MFMA fragment reads for bf16 operands (gfx950).
//
// Tiles are copied from global memory straight into LDS with
// buffer_load_dwordx4 ... lds: each lane moves 16 bytes and the wave writes
// 1 KB of consecutive LDS (from M0), so no VGPRs hold staged data and the copy
// proceeds while the wave computes.  Loads outside a tile's valid rows or
// 16-byte chunks use an offset past the buffer descriptor's range, which the
// hardware returns as zeros, so ragged edges arrive zero-filled.  The copy is
// issued from inline assembly: the compiler then does not know of it and
// inserts none of its own vmcnt waits before later LDS reads (it cannot always
// tell that a copy in flight targets another buffer); completion is the
// caller's business, with wait_vm() before the barrier that publishes a tile.
//
// A tile row of CPR 16-byte chunks (CPR * 8 bf16) is stored unpadded with the
// chunk index XOR-swizzled by a function of the row.  The swizzle keeps both
// fragment reads below free of bank conflicts, for 32 or 64 LDS banks (for
// CPR = 4, only the transpose read):
//  * rows(): lane (r, q) reads row m0 + r, chunk kc + q (one 16-byte read):
//    the MFMA fragment whose k index runs along the row;
//  * cols(): ds_read_b64_tr_b16 pairs that deliver, to lane (r, q), the 8
//    elements of column m0 + r in rows k0 + 8q .. k0 + 8q + 7: the MFMA
//    fragment whose k index runs down the rows.  Within each group of 16
//    lanes the instruction returns to lane i, element e, the (i % 4)-th value
//    read by lane 4e + i / 4, so lane j of the group reads the 4 elements at
//    row k0 + 8q + (j / 4) (+4 for the second read), column m0 + 4 (j % 4).
#pragma once

#include "ssd_common.hpp"

namespace ssd {

typedef __attribute__((address_space(3))) char lds_char;
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Byte offsets at or beyond this value are out of every descriptor's range.
constexpr uint32_t OOB_OFFSET = 0x80000000u;

// Raw buffer descriptor over the 2 GiB that start at `base` (byte offsets,
// stride 0; loads at OOB_OFFSET or beyond return zeros).
__device__ __forceinline__ i32x4 make_rsrc(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{static_cast<int>(a), static_cast<int>((a >> 32) & 0xFFFFu), 0x7FFFFFF0, 0x00020000};
}

// One wave's 16-byte-per-lane copy into LDS at dst + 16 * lane (dst uniform).
__device__ __forceinline__ void dma16(const i32x4& rs, lds_char* dst, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)  // gfx950 assembly: device pass only
  // dst is uniform across the wave but derived from the wave index, so make
  // that explicit for the scalar operand
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst)));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0v), "v"(voff), "s"(rs)
               : "memory", "m0");
#endif
}

// The same with a uniform byte offset added in the instruction's scalar
// offset (voff alone decides whether a lane is out of range).
__device__ __forceinline__ void dma16_so(const i32x4& rs, lds_char* dst, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)  // gfx950 assembly: device pass only
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst)));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(m0v), "v"(voff), "s"(rs),
               "s"(soff)
               : "memory", "m0");
#endif
}

// One wave's copy of 64 16-bit elements into LDS: a sub-dword LDS-direct load
// writes one dword per lane, at dst + 4 * lane, holding the element
// zero-extended (measured on gfx950).  voff at or beyond OOB_OFFSET gives 0.
__device__ __forceinline__ void dma_u16(const i32x4& rs, lds_char* dst, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)  // gfx950 assembly: device pass only
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst)));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_ushort %1, %2, 0 offen lds" ::"s"(m0v), "v"(voff), "s"(rs)
               : "memory", "m0");
#endif
}

// The chunk's Q <= 256 time steps of one 16-bit per-step series (dt of one
// head: element t at byte t * stride from the descriptor's base) into LDS as
// dwords (step t at dst + 4 t), zero past Q.  Every wave issues exactly one
// copy instruction (waves beyond the four a chunk needs repeat a copy, with
// identical data), so that counted waits stay the same in every wave.
template <int NW>
__device__ __forceinline__ void steps_async(lds_char* dst, const i32x4& rs, uint32_t stride, int Q) {
  static_assert(NW >= 4, "four waves cover 256 steps");
  // the lane index passes through opaque_index so that the offsets are
  // recomputed here rather than hoisted out of the caller's loops (where they
  // would hold registers for the whole kernel)
  const int w = wave_id() % 4, t = 64 * w + opaque_index(lane_id());
  dma_u16(rs, dst + 256 * w, t < Q ? static_cast<uint32_t>(t) * stride : OOB_OFFSET);
}

// A buffer descriptor kept as its 64-bit base and built where it is used:
// the base passes through an empty asm first, so that the compiler cannot
// hoist the built descriptor (four SGPRs) out of the loops and keeps only the
// base (two).  For kernels short of SGPRs, whose spills cost v_readlane /
// v_writelane pairs in the loops.
struct LazyRsrc {
  const void* p;
  __device__ __forceinline__ i32x4 get() const {
    uint64_t a = reinterpret_cast<uint64_t>(p);
    asm volatile("" : "+s"(a));
    return i32x4{static_cast<int>(a), static_cast<int>((a >> 32) & 0xFFFFu), 0x7FFFFFF0, 0x00020000};
  }
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t ptr() const {
    uint64_t a = reinterpret_cast<uint64_t>(p);
    asm volatile("" : "+s"(a));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(a), 0, 0x7FFFFFF0, 0x00020000);
  }
};

// The same descriptor in the type the buffer-load builtins take.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_ptr(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFF0, 0x00020000);
}

// The same for an optional output: a null pointer gets an empty range, so
// every access through the descriptor is dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_opt(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, base ? 0x7FFFFFF0 : 0, 0x00020000);
}

__device__ __forceinline__ lds_char* lds_ptr(void* p) { return (lds_char*)p; }

// vmcnt(n) with the other counters left alone: at most n of this wave's
// vector-memory operations (loads, stores, asynchronous copies; they retire
// in issue order) remain outstanding.  The empty asm statements keep the
// compiler from moving memory operations across the wait, so that n counts
// what the source issued before it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070 | 0x0F00);
  __asm__ volatile("" ::: "memory");
}

// Workgroup barrier for LDS data written with ds_write only: waits for this
// wave's LDS operations (lgkmcnt) but not for vector-memory operations, so
// asynchronous tile copies stay in flight across it (__syncthreads' fence
// would wait for them too).  The empty asm statements keep the compiler from
// moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maximum
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

template <int CPR>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CPR <= 2 || CPR >= 32) {
    return 0;
  } else if constexpr (CPR == 4) {
    // 64-byte rows (read with the transpose read only): rows r and r + 2 of a
    // group of four share banks, so they take opposite chunk pairs
    return ((r >> 1) & 1) << 1;
  } else {
    const int b = ((r & 3) << 1) | ((r >> 2) & 1);
    return b ^ (((r >> 3) & 1) * (CPR == 16 ? 8 : 2));
  }
}

template <int CPR>
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return row * (CPR * 16) + ((chunk ^ swz<CPR>(row)) << 4);
}

// Copy rows 0..ROWS-1 of a bf16 matrix into an LDS tile of ROWS x CPR chunks:
// row r starts at byte base + r * ldb of the descriptor; rows >= row_ok and
// chunks >= chunk_ok are zero.  The NW waves of the workgroup share the copy.
template <int ROWS, int CPR, int NW>
__device__ __forceinline__ void tile_async(lds_char* dst, const i32x4& rs, uint32_t base,
                                           uint32_t ldb, int row_ok, int chunk_ok) {
  constexpr int LPI = 64 / CPR;  // rows per wave instruction
  constexpr int NI = ROWS / LPI;
  static_assert(ROWS % LPI == 0, "tile rows");
  const int l = lane_id(), w = wave_id();
  const int rl = l / CPR, pc = l % CPR;
#pragma unroll
  for (int it = 0; it < (NI + NW - 1) / NW; ++it) {
    const int ins = it * NW + w;
    if ((NI % NW) == 0 || ins < NI) {
      const int r = ins * LPI + rl;
      const int c = pc ^ swz<CPR>(r);
      const uint32_t off = (r < row_ok && c < chunk_ok) ? base + static_cast<uint32_t>(r) * ldb + (c << 4) : OOB_OFFSET;
      dma16(rs, dst + ins * 1024, off);
    }
  }
}

// tile_async's per-lane addressing computed once, for a tile that is copied
// many times from sources that differ by a uniform byte offset: each copy then
// costs one compare and one select per instruction.
template <int ROWS, int CPR, int NW>
struct TileLanes {
  static constexpr int LPI = 64 / CPR, NI = ROWS / LPI, PER = (NI + NW - 1) / NW;
  static_assert(ROWS % LPI == 0, "tile rows");
  uint32_t off[PER];  // r * ldb + 16 c, or OOB_OFFSET for chunks >= chunk_ok
  int row[PER];       // r, or ROWS for instructions past the tile
  __device__ __forceinline__ void init(uint32_t ldb, int chunk_ok) {
    const int l = lane_id(), w = wave_id();
    const int rl = l / CPR, pc = l % CPR;
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int ins = it * NW + w;
      const int r = ins * LPI + rl;
      const int c = pc ^ swz<CPR>(r);
      off[it] = c < chunk_ok ? static_cast<uint32_t>(r) * ldb + (c << 4) : OOB_OFFSET;
      row[it] = ((NI % NW) == 0 || ins < NI) ? r : ROWS;
    }
  }
  // rows >= row_ok are zero; the tile's row 0 starts at byte soff
  __device__ __forceinline__ void issue(lds_char* dst, const i32x4& rs, uint32_t soff, int row_ok) const {
    const int w = wave_id();
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int ins = it * NW + w;
      if ((NI % NW) == 0 || ins < NI) dma16_so(rs, dst + ins * 1024, row[it] < row_ok ? off[it] : OOB_OFFSET, soff);
    }
  }
};

// TileLanes' copy with the per-lane offsets recomputed at the issue from an
// opaque lane index, for kernels where keeping them live across a loop would
// spill them (a spilled offset's reload waits for every copy in flight).
template <int ROWS, int CPR, int NW>
__device__ __forceinline__ void tile_issue_fresh(lds_char* dst, const i32x4& rs, uint32_t ldb, int chunk_ok,
                                                 uint32_t soff, int row_ok) {
  constexpr int LPI = 64 / CPR, NI = ROWS / LPI;
  static_assert(ROWS % LPI == 0, "tile rows");
  const int l = opaque_index(lane_id()), w = wave_id();
  const int rl = l / CPR, pc = l % CPR;
#pragma unroll
  for (int it = 0; it < (NI + NW - 1) / NW; ++it) {
    const int ins = it * NW + w;
    if ((NI % NW) == 0 || ins < NI) {
      const int r = ins * LPI + rl;
      const int c = pc ^ swz<CPR>(r);
      const uint32_t off = (c < chunk_ok && r < row_ok) ? static_cast<uint32_t>(r) * ldb + (c << 4) : OOB_OFFSET;
      dma16_so(rs, dst + ins * 1024, off, soff);
    }
  }
}

// Fragment with k along the row: lane (r, q) gets row m0 + r, elements
// 8 (kc + q) .. +7.
template <int CPR>
__device__ __forceinline__ bf16x8 frag_rows(const lds_char* t, int m0, int kc) {
  const int l = lane_id(), r = l & 15, q = l >> 4;
  const int row = m0 + r;
  return *(const __attribute__((address_space(3))) bf16x8*)(t + tile_off<CPR>(row, kc + q));
}

// Fragment with k down the rows: lane (r, q) gets column m0 + r, rows
// k0 + 8q .. k0 + 8q + 7 (m0 a multiple of 16, k0 of 8).
template <int CPR>
__device__ __forceinline__ bf16x8 frag_cols(const lds_char* t, int k0, int m0) {
  const int l = lane_id(), i = l & 15, q = l >> 4;
  const int c = (m0 >> 3) + ((i >> 1) & 1), half = (i & 1) << 3;
  const int r0 = k0 + 8 * q + (i >> 2), r1 = r0 + 4;
  const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)(t + tile_off<CPR>(r0, c) + half));
  const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)(t + tile_off<CPR>(r1, c) + half));
  const short8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// The same reads from per-lane base offsets.  The swizzle only permutes the
// 16-byte chunks inside a row, so for m0 and k0 multiples of 16 and kc a
// multiple of 4 every address of a read is the lane's offset at
// m0 = k0 = kc = 0, XORed with the chunk offset of kc (rows) or m0 (columns),
// plus the row offset of m0 (rows) or k0 (columns): one VALU operation per
// read.  The bases are computed once; a loop body passes them through
// opaque() so that the compiler recomputes the few XORs per iteration
// instead of keeping one register per distinct address alive across the loop.
template <int CPR>
struct RowsAt {
  int b;
};
template <int CPR>
struct ColsAt {
  int b;  // the first transpose read (rows k0 + 8q + i/4); the second reads 4 rows further
};
template <int CPR>
__device__ __forceinline__ RowsAt<CPR> rows_at() {
  const int l = lane_id(), r = l & 15, q = l >> 4;
  return {r * (CPR * 16) + ((q ^ swz<CPR>(r)) << 4)};
}
// Strips (tiles of 32-byte rows that a wave writes from its MFMA output and
// the transpose read consumes) are stored with rows 8..15 of every 16 moved
// four rows on and their two 16-byte halves swapped: byte b of row R is at
// (32 R + b) ^ (0x90 if bit 3 of R is set).  Unswizzled, the transpose read
// (rows 8q + 0..3 per 16-lane group) and the 8-byte row writes meet the same
// banks two ways.
__device__ __forceinline__ int strip_off(int row, int byte) {
  return (row * 32 + byte) ^ (((row >> 3) & 1) * 0x90);
}
template <int CPR>
__device__ __forceinline__ ColsAt<CPR> cols_at() {
  const int l = lane_id(), i = l & 15, q = l >> 4;
  const int half = (i & 1) << 3, ra = 8 * q + (i >> 2);
  if constexpr (CPR == 2) return {strip_off(ra, (((i >> 1) & 1) << 4) + half)};
  return {ra * (CPR * 16) + ((((i >> 1) & 1) ^ swz<CPR>(ra)) << 4) + half};
}
template <int CPR>
__device__ __forceinline__ RowsAt<CPR> opaque(RowsAt<CPR> a) {
  asm volatile("" : "+v"(a.b));
  return a;
}
template <int CPR>
__device__ __forceinline__ ColsAt<CPR> opaque(ColsAt<CPR> a) {
  asm volatile("" : "+v"(a.b));
  return a;
}
template <int CPR>
__device__ __forceinline__ bf16x8 frag_rows(const lds_char* t, int m0, int kc, RowsAt<CPR> a) {
  return *(const __attribute__((address_space(3))) bf16x8*)(t + ((a.b ^ (kc << 4)) + m0 * (CPR * 16)));
}
template <int CPR>
__device__ __forceinline__ bf16x8 frag_cols(const lds_char* t, int k0, int m0, ColsAt<CPR> a) {
  // rows r and r + 4 (r % 8 < 4) differ in the low bit of the swizzle of 8-
  // and 16-chunk rows, not at all for 4- and 32-chunk rows; in a strip row
  // r + 4 is the XOR of row r's offset with 128 (strip_off)
  constexpr int flip = (CPR == 8 || CPR == 16) ? 16 : (CPR == 2 ? 128 : 0);
  constexpr int four_rows = CPR == 2 ? 0 : 4 * CPR * 16;
  const int x = (m0 >> 3) << 4, o = k0 * (CPR * 16);
  const short4_t lo =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(t + ((a.b ^ x) + o)));
  const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)(t + ((a.b ^ (x ^ flip)) + o + four_rows)));
  const short8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// A 16 x 16 block of a tile in the MFMA accumulator layout: lane (r, q) gets
// elements (m0 + 4q + e, n0 + r), e = 0..3, as bf16 pairs {e0 | e1 << 16,
// e2 | e3 << 16}, from one transpose read (lane i of a 16-lane group reads the
// 4 elements at row m0 + 4q + i/4, column n0 + 4 (i % 4)).  m0 and n0 are
// multiples of 16; the per-lane offset is XOR-composed like the fragments'.
template <int CPR>
struct AccAt {
  int b;
};
template <int CPR>
__device__ __forceinline__ AccAt<CPR> acc_at() {
  const int l = lane_id(), i = l & 15, q = l >> 4;
  const int ra = 4 * q + (i >> 2);
  return {ra * (CPR * 16) + ((((i >> 1) & 1) ^ swz<CPR>(ra)) << 4) + ((i & 1) << 3)};
}
template <int CPR>
__device__ __forceinline__ AccAt<CPR> opaque(AccAt<CPR> a) {
  asm volatile("" : "+v"(a.b));
  return a;
}
template <int CPR>
__device__ __forceinline__ u32x2 block_acc(const lds_char* t, int m0, int n0, AccAt<CPR> a) {
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)(t + ((a.b ^ ((n0 >> 3) << 4)) + m0 * (CPR * 16))));
  return __builtin_bit_cast(u32x2, v);
}
// Element e of a block_acc() result, as f32.
__device__ __forceinline__ float acc_elem(const u32x2& v, int e) {
  const uint32_t d = v[e >> 1];
  return __uint_as_float((e & 1) ? (d & 0xFFFF0000u) : (d << 16));
}

// Raw buffer stores of one element at byte offset voff + soff (soff uniform).
// A voff at or beyond OOB_OFFSET is out of the descriptor's range and the
// store is dropped, which predicates stores without branches.
__device__ __forceinline__ void store_f32(__amdgpu_buffer_rsrc_t rs, float v, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, voff, soff, 0);
}
__device__ __forceinline__ void store_b16(__amdgpu_buffer_rsrc_t rs, uint16_t v, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b16(v, rs, voff, soff, 0);
}
// Four consecutive floats at a 16-byte aligned offset as one 16-byte store.
__device__ __forceinline__ void store_f32x4(__amdgpu_buffer_rsrc_t rs, const f4& v, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, voff, soff, 0);
}
// Eight consecutive floats rounded to bf16 as one 16-byte store.
__device__ __forceinline__ void store_bf16x8(__amdgpu_buffer_rsrc_t rs, const float4& a, const float4& b,
                                             uint32_t voff, uint32_t soff) {
  const u32x4 v = {pack_bf16(a.x, a.y), pack_bf16(a.z, a.w), pack_bf16(b.x, b.y), pack_bf16(b.z, b.w)};
  __builtin_amdgcn_raw_buffer_store_b128(v, rs, voff, soff, 0);
}

// One element (row, col) of a swizzled tile, as f32.
template <int CPR>
__device__ __forceinline__ float tile_elem(const lds_char* t, int row, int col) {
  const uint16_t v =
      *(const __attribute__((address_space(3))) uint16_t*)(t + tile_off<CPR>(row, col >> 3) + ((col & 7) << 1));
  return bf16_bits_to_f32(v);
}

// Scheduling groups (AMDGPU sched_group_barrier): the next N LDS reads, or N
// MFMAs, of the enclosing scheduling region are placed here, in program
// order of the groups.  Used to issue all of a phase's fragment reads before
// its MFMAs, so that their latencies overlap.
template <int N>
__device__ __forceinline__ void sched_ds_reads() {
  __builtin_amdgcn_sched_group_barrier(0x100, N, 0);
}
template <int N>
__device__ __forceinline__ void sched_mfmas() {
  __builtin_amdgcn_sched_group_barrier(0x008, N, 0);
}

// Sum over each row of 16 lanes (lanes sharing q), complete in lane r = 15
// (DPP row shifts, zero-filled at the row start).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_sum16(float v) {
  v = dpp_add<0x111>(v);  // row_shr:1
  v = dpp_add<0x112>(v);  // row_shr:2
  v = dpp_add<0x114>(v);  // row_shr:4
  return dpp_add<0x118>(v);  // row_shr:8
}

// Inclusive scan over the 64 lanes of a wave: shifts within rows of 16, then
// row_bcast15 / row_bcast31 carry each row's total into the following rows
// (DPP; zero where a lane has no source).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add_rows(float v) {
  return v + __builtin_bit_cast(float,
                                __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, true));
}
__device__ __forceinline__ float wave_scan(float v) {
  v = dpp_add<0x111>(v);
  v = dpp_add<0x112>(v);
  v = dpp_add<0x114>(v);
  v = dpp_add<0x118>(v);
  v = dpp_add_rows<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  return dpp_add_rows<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
}

// s (within-chunk inclusive cumsum of dt A) and dt for t < Q, from the dt bits
// copied to LDS (one dword per step; lane l reads t = 4l .. 4l+3); every wave
// computes the whole scan and waves 0..3 each write a quarter.
__device__ __forceinline__ void scan_store(const uint32_t* dtb_lds, float A, float* s_out, float* dt_out) {
  const int l = opaque_index(lane_id()), w = wave_id();  // recomputed, as in steps_async
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

// Write two MFMA tiles (lane element e at row j = 4q + e, column i = 16 tt + r)
// into a wave strip as bf16 [i][j] (32 rows i of 16 columns j).
__device__ __forceinline__ void put_strip(lds_char* strip, const f4 (&v)[2]) {
  const int l = lane_id(), r = l & 15, q = l >> 4;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
    *(__attribute__((address_space(3))) u32x2*)(strip + strip_off(16 * tt + r, 8 * q)) =
        u32x2{pack_bf16(v[tt][0], v[tt][1]), pack_bf16(v[tt][2], v[tt][3])};
}

}  // namespace ssd
