// Device-side building blocks shared by the gfx950 kernels of the absorbed
// Gated MLA library: vector types, MFMA wrappers, LDS transpose reads, direct
// global->LDS copies, the latent-tile swizzle and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define MLA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;

// D = A * B + C on a 16x16x32 bf16 MFMA.  Lane l holds A row (l % 16),
// k = 8 * (l / 16) + 0..7; B column (l % 16) with the same k; C/D column
// (l % 16), register i at row 4 * (l / 16) + i.
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// XOR swizzle of the 16-byte chunks of a latent row held in LDS.  It keeps
// both access patterns of a 32-row tile free of bank conflicts (measured with
// the LDS bank-conflict counter on gfx950, where simpler row XORs leave one
// or the other pattern 2-way conflicted):
//  * ds_read_b128 of one chunk from 16 consecutive rows (score operand), and
//  * ds_read_b64_tr_b16 of 4 rows x 2 chunks per 16-lane group (value
//    operand, both 8-byte halves of each chunk).
template <int R>
__device__ __host__ __forceinline__ constexpr int chunk_swizzle(int s) {
  if constexpr (R / 8 >= 16) {
    return (s & 8) ^ ((s & 7) << 1) ^ ((s >> 3) & 1);
  } else if constexpr (R / 8 == 4) {
    return (((s >> 2) & 1) << 1) | ((s >> 3) & 1);
  } else {
    return 0;
  }
}

// The chunk swizzle of the single-wave prefill tiles (32x32x16 operands):
// row bits 0-1 and 2-3 exchanged, f(4a + e) = 4e + a, applied to the low 4
// bits of the chunk index.  Bank-conflict free for
//  * ds_read_b128 of one chunk from 16 consecutive rows (score operand), and
//  * ds_read_b64_tr_b16 where each 32-lane half reads 4 consecutive rows x
//    4 consecutive chunks (value operand: f's high bits differ across the 4
//    rows, the chunk's low bits across the 4 chunks).
// (chunk_swizzle maps such a 4 x 4 block onto 8 bank groups only.)
template <int R>
__device__ __host__ __forceinline__ constexpr int chunk_swizzle_x(int s) {
  if constexpr (R / 8 >= 16) {
    return ((s & 3) << 2) | ((s >> 2) & 3);
  } else {
    return 0;
  }
}

// SW = 0: chunk_swizzle, SW = 1: chunk_swizzle_x.
template <int R, int SW>
__device__ __host__ __forceinline__ constexpr int tile_swizzle(int s) {
  if constexpr (SW == 1) {
    return chunk_swizzle_x<R>(s);
  } else {
    return chunk_swizzle<R>(s);
  }
}

// Byte offset of (row s, logical 16-byte chunk L) in a swizzled tile.
template <int R>
__device__ __forceinline__ int tile_off(int s, int L) {
  return s * (R * 2) + ((L ^ chunk_swizzle<R>(s)) << 4);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const MLA_LDS char* p) {
  return *(const MLA_LDS bf16x8*)p;
}

// ds_read_b64_tr_b16: within each 16-lane group the 16 lanes' 8-byte chunks
// form a 4 x 16 matrix (lane 4e + q supplies row e, columns 4q..4q+3) and
// lane i receives column i (four rows).
__device__ __forceinline__ bf16x4 lds_read_tr16(const MLA_LDS char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)p);
}

__device__ __forceinline__ bf16x8 cat4(const bf16x4& lo, const bf16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Raw buffer descriptor (gfx9 layout) over `bytes` bytes at `base`: stride 0,
// so a lane whose offset is at or past `bytes` reads zeros.  Held in SGPRs.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, unsigned bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  // callers pass wave-uniform values; readfirstlane keeps the descriptor in
  // SGPRs even where the compiler cannot prove that
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((unsigned)a);
  r[1] = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32) & 0xFFFFu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000u;
  return r;
}

// Direct 16-byte buffer -> LDS copy at byte offset voff: lane l's 16 bytes
// land at lds_base + 16*l (lds_base wave-uniform); out-of-range lanes write
// zeros.  Completion is tracked by vmcnt, and callers wait for it explicitly
// with wait_vmcnt<N>() before the barrier that publishes a tile.
//
// The copy is issued from inline assembly on purpose.  When the compiler sees
// an LDS-DMA load it cannot tell which LDS bytes it writes, so it puts
// vmcnt(0) in front of the next LDS read of any address, which drains every
// prefetch in flight and serialises the copy of tile n+1 with the reads of
// tile n.  Hidden in assembly, the copy is ordered only by the explicit waits
// and barriers of the pipeline (the memory clobber keeps the compiler from
// moving LDS accesses across it).  M0 is written here, with the one wait
// state the hardware needs between an M0 write and an LDS-DMA instruction.
// (The compiler reserves M0 and warns about the clobber; no other code in
// these kernels reads M0, since gfx9 LDS instructions do not use it.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void buf2lds16(const u32x4& rs, unsigned voff, MLA_LDS char* lds_base) {
  const unsigned m0v = (unsigned)(uintptr_t)lds_base;
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rs), "s"(m0v)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// Workgroup barrier without a memory fence.  __syncthreads() also waits for
// every outstanding global access (vmcnt(0)), which would drain the tile
// prefetches in flight; here the LDS hand-off is ordered explicitly instead:
// a wave's own tile copies are waited for with wait_vmcnt<N>() before the
// barrier, and a wave's LDS reads have returned (their values are consumed by
// MFMAs) before it reaches the barrier that lets the stage be refilled.  The
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Scalar (SMEM) load of a wave-uniform int.  A plain load of a value the
// compiler cannot prove read-only becomes a vector load, and waiting for it
// (vmcnt) would also wait for every LDS-DMA tile copy in flight.  The SMEM
// load is tracked by lgkmcnt instead; it waits for itself before returning.
__device__ __forceinline__ int sload_i32(const int* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  // readfirstlane returns int: widen through unsigned, or a low word with
  // bit 31 set would sign-extend over the high word
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)a);
  const uint64_t s = ((uint64_t)hi << 32) | (uint64_t)lo;
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(s) : "memory");
  return v;
}

__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

// s_waitcnt vmcnt(N) leaving the other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// max of finite-or-(-inf) floats as one v_max / v_max3.  fmaxf must quiet
// signalling NaNs, so the compiler puts a canonicalising v_max x, x in front
// of every operand it cannot prove canonical (MFMA and LDS results); scores
// are never NaN, so the plain instruction gives the same value.
__device__ __forceinline__ float max_nn(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_nn(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// max of the 8 values of two C fragments (never NaN)
__device__ __forceinline__ float max8_nn(const f32x4& a, const f32x4& b) {
  return max3_nn(max3_nn(a[0], a[1], a[2]), max3_nn(a[3], b[0], b[1]), max3_nn(b[2], b[3], -INFINITY));
}

// Value of x from the lane in the other half of the wave (l ^ 32) combined
// with x itself, via v_permlane32_swap.
__device__ __forceinline__ float xhalf_max(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return max_nn(__builtin_bit_cast(float, (unsigned)p[0]), __builtin_bit_cast(float, (unsigned)p[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)p[0]) + __builtin_bit_cast(float, (unsigned)p[1]);
}

// Combine x over the four lanes l, l^16, l^32, l^48 (one MFMA column);
// col_max takes values that are never NaN.
__device__ __forceinline__ float col_max(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = max_nn(__builtin_bit_cast(float, (unsigned)p[0]), __builtin_bit_cast(float, (unsigned)p[1]));
  return xhalf_max(x);
}
__device__ __forceinline__ float col_sum(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __builtin_bit_cast(float, (unsigned)p[0]) + __builtin_bit_cast(float, (unsigned)p[1]);
  return xhalf_sum(x);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// (v_rcp_f32, about 1 ulp: the gated value is rounded to bf16 anyway; a
// correctly rounded divide costs a dozen instructions more per element)
__device__ __forceinline__ float sigmoidf_(float g) { return __builtin_amdgcn_rcpf(1.0f + fast_exp2(-g * kLog2e)); }

// Two 4-value C fragments (scaled) -> one bf16 MFMA operand (k slots 0-3
// from lo, 4-7 from hi), round-to-nearest-even.
__device__ __forceinline__ bf16x8 pack44(const f32x4& lo, const f32x4& hi, float s) {
  bf16x8 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    r[p] = (bf16)(lo[p] * s);
    r[p + 4] = (bf16)(hi[p] * s);
  }
  return r;
}

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }

}  // namespace mla
