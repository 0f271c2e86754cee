// Building blocks of the one-wave-per-SIMD bf16 attention kernels on gfx950
// (prefill and decode at r >= 256): v_mfma_f32_32x32x16_bf16 issued from
// inline assembly with explicit hazard handling, and the LDS operand
// addressing of a 32-key latent tile for the two products of page
// "Gated MLA（矩阵吸收版）", section 完整计算流（四步） steps 2 and 3 in their
// transposed form (one output column per lane pair):
//   S^T  = c_tile . q_abs^T          32 keys x 32 columns, fp32
//   O^T += c_tile^T . P^T             [r x 32] fp32
#pragma once

#include "attn_core.h"

namespace mla {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// v_mfma_f32_32x32x16_bf16: D = A * B + C.  Lane l holds A row (l % 32),
// k = 8 (l / 32) + 0..7; B column (l % 32) with the same k; C/D column
// (l % 32), register i at row 8 (i / 4) + 4 (l / 32) + i % 4.
//
// Every product of these kernels is issued from inline assembly, with the
// accumulator's register file fixed by the constraint: O^T in accumulation
// registers ("a"), the score, absorb and epilogue chains in VGPRs ("v").
// Through the builtin, the compiler selects the accumulation-register form
// for every MFMA of a one-wave-per-SIMD kernel, so the score accumulator
// competes with the 256 registers of O^T, and its allocator then spills O^T
// at every loop header.  The compiler does not see these MFMAs, so the code
// around them keeps each hazard explicit:
//  * a chain starts with the zero-accumulator form (no write of the
//    accumulator precedes it) or follows settle_*() after a VALU write;
//  * chained products accumulate into the exact same registers, which the
//    hardware forwards without wait states;
//  * a result is read by VALU or memory instructions only after settle_*()
//    (24 wait states, above what an XDL write followed by a read needs);
//  * an operand written by a VALU instruction is pinned right after it is
//    formed (an empty asm that takes it as an in-out operand, so the compiler
//    cannot sink its computation towards the product) and separated from
//    its product by operand_gap() (2 wait states); operands loaded from
//    memory are ordered by the lgkmcnt / vmcnt waits the compiler puts
//    before the asm.
__device__ __forceinline__ void mfma32v_first(f32x16& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
// chain start from an accumulator held in other registers (init is only read)
__device__ __forceinline__ void mfma32v_init(f32x16& c, const bf16x8& a, const bf16x8& b, const f32x16& init) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(c) : "v"(a), "v"(b), "v"(init));
}
__device__ __forceinline__ void mfma32v(f32x16& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32a(f32x16& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void settle_v(f32x16& c) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c));
}
__device__ __forceinline__ void wait_states_24() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }
__device__ __forceinline__ void operand_gap() { asm volatile("s_nop 1" ::: "memory"); }
// Pins an accumulator in its accumulation registers at this point of the
// instruction stream (orders compiler reads and writes of it against the
// volatile asm around).
__device__ __forceinline__ void pin_a(f32x16& c) { asm volatile("" : "+a"(c)); }

// c = 0 in accumulation registers, as the product of zero operands: every
// block is then a value of its own (one shared zero constant would stay live
// beside O^T), and the value products that follow read it as their
// accumulator straight from the matrix pipe.
__device__ __forceinline__ void zero_a(f32x16& c, const bf16x8& z) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=&a"(c) : "v"(z));
}

// c *= alpha on accumulation registers, element by element in assembly so
// the accumulator never becomes a VGPR value (a compiler multiply would copy
// all of O^T through VGPRs and break its allocation).
__device__ __forceinline__ void scale_acc(f32x16& c, float alpha) {
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    float tmp;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(c[k]), "=&v"(tmp)
                 : "v"(alpha));
  }
}

// 8 fp32 values (scaled) -> bf16 MFMA operand, round-to-nearest-even.
__device__ __forceinline__ bf16x8 pack8(const f32x16& v, int base, float s) {
  bf16x8 r;
#pragma unroll
  for (int p = 0; p < 8; ++p) r[p] = (bf16)(v[base + p] * s);
  return r;
}

// a compile-time flag passed to a generic lambda (one specialised body each)
template <bool V>
struct BoolTag {
  static constexpr bool value = V;
};

typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));

// acc + the sum of the 8 bf16 values of p: four v_dot2 against (1, 1).  The
// softmax denominator then adds the bf16 P that the value products use, in
// half the instructions of an fp32 sum of the unrounded exponentials.
__device__ __forceinline__ float sum8_bf16(const bf16x8& p, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 6, 7), one, acc, false);
}

template <int R>
struct SoloAttn {
  static constexpr int NKK = R / 16;  // score k-blocks (16 latent dims)
  static constexpr int NLB = R / 32;  // 32-dim latent blocks of O^T
  static constexpr int ROWB = R * 2;
  static_assert(R / 8 >= 16 && R % 128 == 0, "solo layout needs r >= 256");

  // Operand addresses inside a tile (XOR chunk swizzle folded in):
  //  * score operand of k-block kk: key row l % 32, chunk 2kk + l / 32, at
  //    qb[kk & 7] + 256 (kk >> 3);
  //  * value operand n = NLB kb + t of latent block t, key block kb (keys
  //    16kb + ...), two transposing reads: rows 16kb + 4 (l / 32) + e (+ 8), chunk
  //    4t + 2 ((l / 16) & 1) + (l % 4) / 2, at vb[4j + (t & 3)] + 256 (t >> 2)
  //    + 16 ROWB kb.
  int qb[8], vb[8];

  __device__ __forceinline__ void init_addressing(int lane) {
    const int l32 = lane & 31, hh = lane >> 5;
    const int xs = chunk_swizzle_x<R>(l32);
#pragma unroll
    for (int u = 0; u < 8; ++u) qb[u] = l32 * ROWB + (((2 * u + hh) ^ xs) << 4);
    const int g = lane >> 4, i = lane & 15, e = i >> 2, q = i & 3;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = 4 * (g >> 1) + e + 8 * j;
      const int xr = chunk_swizzle_x<R>(row);
#pragma unroll
      for (int u = 0; u < 4; ++u) vb[4 * j + u] = row * ROWB + (((4 * u + 2 * (g & 1) + (q >> 1)) ^ xr) << 4) + (q & 1) * 8;
    }
  }

  __device__ __forceinline__ bf16x8 score_operand(const MLA_LDS char* tile, int kk) const {
    return lds_read_b128(tile + qb[kk & 7] + 256 * (kk >> 3));
  }
  __device__ __forceinline__ bf16x8 value_operand(const MLA_LDS char* tile, int n) const {
    // n = NLB kb + t
    const int t = n % NLB, kb = n / NLB;
    const MLA_LDS char* p = tile + 256 * (t >> 2) + 16 * ROWB * kb;
    return cat4(lds_read_tr16(p + vb[t & 3]), lds_read_tr16(p + vb[4 + (t & 3)]));
  }
};

}  // namespace mla
