// bf16 GEMM for the projections around the absorbed core (page "Gated MLA
// （矩阵吸收版）", section 完整计算流（四步）: the query low-rank path of step 1,
// the latent down-projection of section 低秩压缩, the gate and the output
// projection of step 4).  Every projection is a linear layer
//
//   Y[m, n] = sum_k X[m, k] * W[n, k]        X [M, K], W [N, K], Y [M, N]
//
// (row-major, K contiguous in both operands, the weight laid out as
// out_features x in_features), bf16 storage with fp32 accumulation.  Rows
// may be strided (lda, ldw, ldy) and blockIdx.y indexes a batch (per-head
// products of the backward).
//
// Workgroup: 4 waves, a 128 (n) x 128 (m) tile of Y^T, 64-wide k tiles in
// two LDS stages.  The MFMA computes Y^T = W X^T, so its A operand rows are
// W rows and its B operand columns are X rows, both read from K-contiguous
// LDS rows with 16-byte reads, and each lane's C fragment holds four
// consecutive n of one m: the stores are 8 bytes wide.  Wave (wn, wm) owns a
// 64 x 64 block of the tile: 4 x 4 MFMA tiles.
//
// LDS rows are 128 bytes (64 bf16); the 16-byte chunk c of row s is stored at
// chunk c ^ ((s >> 1) & 7), which spreads the 16 rows read by one 16-lane
// group over all 64 banks.  Tiles are copied from global memory straight into
// LDS (buffer loads with the LDS bit); rows past M or N read as zeros.
#pragma once

#include "common.h"

namespace mla {

struct GemmArgs {
  const bf16* x;  // [M, K], rows lda apart
  const bf16* w;  // [N, K], rows ldw apart
  bf16* y;        // [M, N], rows ldy apart
  int M, N, K;    // K % 8 == 0; a last partial k tile reads zeros past K
  int tiles_n;    // ceil(N / 128)
  int lda, ldw, ldy;
  long long bsx, bsw, bsy;  // element offsets between the batches of blockIdx.y
  float alpha;              // Y = alpha X W^T
};

constexpr int kGemmTile = 128;
constexpr int kGemmKT = 64;
constexpr int kGemmTileBytes = kGemmTile * kGemmKT * 2;  // 16 KiB per operand per stage

__device__ __forceinline__ int gemm_chunk(int s, int c) { return c ^ ((s >> 1) & 7); }

// Copies rows [row0, row0 + 128) x k [k0, k0 + 64) of a K-contiguous
// operand into a swizzled LDS tile.  Copy i (1 KiB = 8 rows) is issued by
// wave i % 4; lane l of a copy fills LDS bytes 16 l .. of it, which is row
// 8 i + l / 8, physical chunk l % 8.
__device__ __forceinline__ void gemm_copy(const bf16* __restrict__ base, int rows_total, int row0, int ld,
                                          int K, int k0, MLA_LDS char* tile, int w) {
  unsigned ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  int rows = rows_total - row0;
  rows = rows > kGemmTile ? kGemmTile : rows;
  // the descriptor ends at the last valid row's row start + ld: rows past it read as zeros
  const u32x4 rs = make_rsrc(base + (size_t)row0 * ld, (unsigned)((size_t)(rows > 0 ? rows : 0) * ld * 2));
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int i = w + 4 * c;  // copy index 0..15
    const int s = 8 * i + (int)(ln >> 3);
    const int logical = gemm_chunk(s, (int)(ln & 7));
    const int k = k0 + 8 * logical;  // columns past K read as zeros
    const unsigned voff = k < K ? (unsigned)(((size_t)s * ld + k) * 2) : 0xFFFFFFF0u;
    buf2lds16(rs, voff, tile + i * 1024);
  }
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
mla_gemm_nt(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * 2 * kGemmTileBytes];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;  // [stage][W tile, X tile]

  const int tn = blockIdx.x % a.tiles_n, tm = blockIdx.x / a.tiles_n;
  const int n0 = tn * kGemmTile, m0 = tm * kGemmTile;
  const bf16* __restrict__ X = a.x + (size_t)blockIdx.y * a.bsx;
  const bf16* __restrict__ W = a.w + (size_t)blockIdx.y * a.bsw;
  bf16* __restrict__ Y = a.y + (size_t)blockIdx.y * a.bsy;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, kq = lane >> 4;
  const int wn = w & 1, wm = w >> 1;  // this wave's 64 x 64 block
  const int nk = (a.K + kGemmKT - 1) / kGemmKT;

  auto stage_w = [&](int st) { return smem + st * 2 * kGemmTileBytes; };
  auto stage_x = [&](int st) { return smem + st * 2 * kGemmTileBytes + kGemmTileBytes; };

  gemm_copy(W, a.N, n0, a.ldw, a.K, 0, stage_w(0), w);
  gemm_copy(X, a.M, m0, a.lda, a.K, 0, stage_x(0), w);

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{};

  // operand byte offsets inside a tile: row (64 wn/wm + 16 t + l16), logical
  // chunk 4 ks + kq of the 64-wide k tile
  auto off = [&](int row, int chunk) { return row * 128 + (gemm_chunk(row, chunk) << 4); };

  for (int kt = 0; kt < nk; ++kt) {
    wait_vmcnt<0>();
    wg_barrier();  // tile kt visible; every wave is done with tile kt-1
    if (kt + 1 < nk) {
      gemm_copy(W, a.N, n0, a.ldw, a.K, (kt + 1) * kGemmKT, stage_w((kt + 1) & 1), w);
      gemm_copy(X, a.M, m0, a.lda, a.K, (kt + 1) * kGemmKT, stage_x((kt + 1) & 1), w);
    }
    const MLA_LDS char* tw = stage_w(kt & 1);
    const MLA_LDS char* tx = stage_x(kt & 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        fa[t] = lds_read_b128(tw + off(64 * wn + 16 * t + l16, 4 * ks + kq));
        fb[t] = lds_read_b128(tx + off(64 * wm + 16 * t + l16, 4 * ks + kq));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(fa[i], fb[j], acc[i][j]);
    }
  }

  // C fragment (i, j): rows n0 + 64 wn + 16 i + 4 kq + e, column m0 + 64 wm + 16 j + l16
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + 64 * wm + 16 * j + l16;
    if (m >= a.M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + 64 * wn + 16 * i + 4 * kq;
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (bf16)(acc[i][j][e] * a.alpha);
      bf16* dst = Y + (size_t)m * a.ldy + n;
      if (n + 3 < a.N) {
        *(bf16x4*)dst = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < a.N) dst[e] = v[e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The same product with a 256 x 256 tile of Y^T per workgroup of 8 waves
// (each wave 128 n x 64 m: 8 x 4 MFMA tiles), for products with enough
// tiles to fill the chip.  Per k-step a wave reads 12 operand fragments for 32
// MFMAs (the 128 x 128 kernel: 8 for 16), and every staged byte serves twice
// the FLOPs.  Two 64 KiB stages, one workgroup per CU.
constexpr int kGemmBig = 256;

__device__ __forceinline__ void gemm_copy_big(const bf16* __restrict__ base, int rows_total, int row0, int ld, int K,
                                              int k0, MLA_LDS char* tile, int w) {
  unsigned ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  int rows = rows_total - row0;
  rows = rows > kGemmBig ? kGemmBig : rows;
  const u32x4 rs = make_rsrc(base + (size_t)row0 * ld, (unsigned)((size_t)(rows > 0 ? rows : 0) * ld * 2));
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int i = w + 8 * c;  // copy index 0..31, 8 rows each
    const int s = 8 * i + (int)(ln >> 3);
    const int logical = gemm_chunk(s, (int)(ln & 7));
    const int k = k0 + 8 * logical;
    const unsigned voff = k < K ? (unsigned)(((size_t)s * ld + k) * 2) : 0xFFFFFFF0u;
    buf2lds16(rs, voff, tile + i * 1024);
  }
}

__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
mla_gemm_nt_big(GemmArgs a) {
  constexpr int TB = kGemmBig * kGemmKT * 2;  // 32 KiB per operand per stage
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * 2 * TB];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;  // [stage][W tile, X tile]

  const int tn = blockIdx.x % a.tiles_n, tm = blockIdx.x / a.tiles_n;
  const int n0 = tn * kGemmBig, m0 = tm * kGemmBig;
  const bf16* __restrict__ X = a.x + (size_t)blockIdx.y * a.bsx;
  const bf16* __restrict__ W = a.w + (size_t)blockIdx.y * a.bsw;
  bf16* __restrict__ Y = a.y + (size_t)blockIdx.y * a.bsy;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, kq = lane >> 4;
  const int wn = w & 1, wm = w >> 1;  // this wave's 128 (n) x 64 (m) block
  const int nk = (a.K + kGemmKT - 1) / kGemmKT;

  auto stage_w = [&](int st) { return smem + st * 2 * TB; };
  auto stage_x = [&](int st) { return smem + st * 2 * TB + TB; };

  gemm_copy_big(W, a.N, n0, a.ldw, a.K, 0, stage_w(0), w);
  gemm_copy_big(X, a.M, m0, a.lda, a.K, 0, stage_x(0), w);

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{};

  auto off = [&](int row, int chunk) { return row * 128 + (gemm_chunk(row, chunk) << 4); };

  for (int kt = 0; kt < nk; ++kt) {
    wait_vmcnt<0>();
    wg_barrier();  // tile kt visible; every wave is done with tile kt-1
    if (kt + 1 < nk) {
      gemm_copy_big(W, a.N, n0, a.ldw, a.K, (kt + 1) * kGemmKT, stage_w((kt + 1) & 1), w);
      gemm_copy_big(X, a.M, m0, a.lda, a.K, (kt + 1) * kGemmKT, stage_x((kt + 1) & 1), w);
    }
    const MLA_LDS char* tw = stage_w(kt & 1);
    const MLA_LDS char* tx = stage_x(kt & 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 fa[8], fb[4];
#pragma unroll
      for (int t = 0; t < 8; ++t) fa[t] = lds_read_b128(tw + off(128 * wn + 16 * t + l16, 4 * ks + kq));
#pragma unroll
      for (int t = 0; t < 4; ++t) fb[t] = lds_read_b128(tx + off(64 * wm + 16 * t + l16, 4 * ks + kq));
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(fa[i], fb[j], acc[i][j]);
    }
  }

  // C fragment (i, j): rows n0 + 128 wn + 16 i + 4 kq + e, column m0 + 64 wm + 16 j + l16
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + 64 * wm + 16 * j + l16;
    if (m >= a.M) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = n0 + 128 * wn + 16 * i + 4 * kq;
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (bf16)(acc[i][j][e] * a.alpha);
      bf16* dst = Y + (size_t)m * a.ldy + n;
      if (n + 3 < a.N) {
        *(bf16x4*)dst = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < a.N) dst[e] = v[e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// C[z][m][n] = sum_k A[k][m] B[k][n] for the weight gradients of the
// backward (the reduction runs over token rows): A and B are row-major with
// the m / n index contiguous (rows lda / ldb apart, batch z at element
// offsets bsa / bsb), C is fp32 [M, N] per batch (written, not added).
// Workgroup: 4 waves, a 128 x 128 tile of C, 64-row k tiles in two LDS
// stages, each wave 64 x 64.  Both MFMA operands need 8 consecutive k per
// lane, i.e. columns of the stored tiles: they come from transposing
// ds_read_b64_tr_b16 reads.  Tiles are copied from global memory with
// LDS-DMA buffer loads; every column of the tile is read, also past M or N
// (inside the allocation, whose byte size bounds the descriptor, those bytes
// only reach accumulators that are not stored), and k rows past K read as
// zeros.
struct GemmTNArgs {
  const bf16* a;
  const bf16* b;
  float* c;
  int M, N, K;
  int lda, ldb;
  long long bsa, bsb, bsc;
  unsigned a_bytes, b_bytes;  // allocation sizes from the a / b pointers
  int tiles_n;
};

// The k tiles of these products hold 64 token rows of WIDTH (128 or 256)
// columns, row pitch 2 WIDTH bytes.  A transposing read takes 8 bytes of
// 16 rows (8 kq + e, e < 4) at the same columns, and every row of the tile
// starts on bank 0: unswizzled, those 16 rows share 8 banks.  The 16-byte
// chunk L of row s is therefore stored at chunk L ^ gemm_tn_swz(s), an even
// value (the two chunks of a 16-column fragment stay one aligned pair) that
// takes 8 different values over the rows one half-wave reads, so its 32
// lanes cover all 64 banks.
__device__ __forceinline__ int gemm_tn_swz(int s) { return 2 * ((s & 3) | (((s >> 3) & 1) << 2)); }

// Rows k0 .. k0+63 x columns col0 .. col0+WIDTH-1 of a row-major operand
// into a swizzled LDS tile.  Copy i (1 KiB) covers 1024 / (2 WIDTH) rows
// and is issued by wave i % NW; lane l's 16 bytes land at byte 16 l of the
// copy, the row's physical chunk l % (WIDTH / 8), so the lane fetches the
// logical chunk that the swizzle puts there.  k rows past K read as zeros.
template <int WIDTH, int NW>
__device__ __forceinline__ void gemm_tn_copy(const bf16* __restrict__ base, unsigned bytes, int ld, int K, int k0,
                                             long long col0, MLA_LDS char* tile, int w) {
  constexpr int CPR = WIDTH / 8;     // chunks per row
  constexpr int RPC = 64 / CPR;      // rows per copy
  constexpr int COPIES = 64 / RPC;   // copies per tile
  static_assert(COPIES % NW == 0, "copies split evenly over the waves");
  unsigned ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  const u32x4 rs = make_rsrc(base, bytes);
#pragma unroll
  for (int c = 0; c < COPIES / NW; ++c) {
    const int i = w + NW * c;
    const int row = RPC * i + (int)(ln / CPR);
    const int logical = (int)(ln % CPR) ^ gemm_tn_swz(row);
    const int k = k0 + row;
    const unsigned voff = k < K ? (unsigned)((((long long)k * ld) + col0 + 8 * logical) * 2) : 0xFFFFFFF0u;
    buf2lds16(rs, voff, tile + i * 1024);
  }
}

// Operand fragment for columns col .. col+15 (col a multiple of 16) and the
// k-step's 32 rows: lane l gets rows 32 ks + 8 (l/16) + 0..7 of column
// col + l % 16 (two transposing reads of four rows each).
template <int WIDTH>
__device__ __forceinline__ bf16x8 gemm_tn_operand(const MLA_LDS char* tile, int ks, int col, int l16, int kq) {
  const int e = l16 >> 2, q = l16 & 3;
  const int r0 = 32 * ks + 8 * kq + e, r1 = r0 + 4;
  const int lc = (col >> 3) + (q >> 1), half = (q & 1) * 8;
  const MLA_LDS char* p0 = tile + r0 * (2 * WIDTH) + ((lc ^ gemm_tn_swz(r0)) << 4) + half;
  const MLA_LDS char* p1 = tile + r1 * (2 * WIDTH) + ((lc ^ gemm_tn_swz(r1)) << 4) + half;
  return cat4(lds_read_tr16(p0), lds_read_tr16(p1));
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
mla_gemm_tn(GemmTNArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * 2 * kGemmTileBytes];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;
  const int tn = blockIdx.x % a.tiles_n, tm = blockIdx.x / a.tiles_n;
  const int n0 = tn * kGemmTile, m0 = tm * kGemmTile;
  const long long ca = (long long)blockIdx.y * a.bsa + m0, cb = (long long)blockIdx.y * a.bsb + n0;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, kq = lane >> 4;
  const int wn = w & 1, wm = w >> 1;
  const int nk = (a.K + kGemmKT - 1) / kGemmKT;
  auto stage_a = [&](int st) { return smem + st * 2 * kGemmTileBytes; };
  auto stage_b = [&](int st) { return smem + st * 2 * kGemmTileBytes + kGemmTileBytes; };

  gemm_tn_copy<kGemmTile, 4>(a.a, a.a_bytes, a.lda, a.K, 0, ca, stage_a(0), w);
  gemm_tn_copy<kGemmTile, 4>(a.b, a.b_bytes, a.ldb, a.K, 0, cb, stage_b(0), w);
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{};

  for (int kt = 0; kt < nk; ++kt) {
    wait_vmcnt<0>();
    wg_barrier();
    if (kt + 1 < nk) {
      gemm_tn_copy<kGemmTile, 4>(a.a, a.a_bytes, a.lda, a.K, (kt + 1) * kGemmKT, ca, stage_a((kt + 1) & 1), w);
      gemm_tn_copy<kGemmTile, 4>(a.b, a.b_bytes, a.ldb, a.K, (kt + 1) * kGemmKT, cb, stage_b((kt + 1) & 1), w);
    }
    const MLA_LDS char* ta = stage_a(kt & 1);
    const MLA_LDS char* tb = stage_b(kt & 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        fa[t] = gemm_tn_operand<kGemmTile>(ta, ks, 64 * wm + 16 * t, l16, kq);
        fb[t] = gemm_tn_operand<kGemmTile>(tb, ks, 64 * wn + 16 * t, l16, kq);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(fa[i], fb[j], acc[i][j]);
    }
  }
  // C fragment (i, j): rows m0 + 64 wm + 16 i + 4 kq + e, column n0 + 64 wn + 16 j + l16
  float* C = a.c + (size_t)blockIdx.y * a.bsc;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 64 * wn + 16 * j + l16;
      if (n >= a.N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 64 * wm + 16 * i + 4 * kq + e;
        if (m < a.M) C[(size_t)m * a.N + n] = acc[i][j][e];
      }
    }
}

// The same product with a 256 x 256 tile of C per workgroup of 8 waves, each
// wave 128 (m) x 64 (n): 8 x 4 MFMA tiles, 12 operand fragments per 32
// MFMAs.  Two 64 KiB stages, one workgroup per CU.
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
mla_gemm_tn_big(GemmTNArgs a) {
  constexpr int TB = kGemmBig * kGemmKT * 2;  // 32 KiB per operand per stage
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * 2 * TB];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;
  const int tn = blockIdx.x % a.tiles_n, tm = blockIdx.x / a.tiles_n;
  const int n0 = tn * kGemmBig, m0 = tm * kGemmBig;
  const long long ca = (long long)blockIdx.y * a.bsa + m0, cb = (long long)blockIdx.y * a.bsb + n0;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, kq = lane >> 4;
  const int wn = w & 3, wm = w >> 2;  // this wave's 128 (m) x 64 (n) block
  const int nk = (a.K + kGemmKT - 1) / kGemmKT;
  auto stage_a = [&](int st) { return smem + st * 2 * TB; };
  auto stage_b = [&](int st) { return smem + st * 2 * TB + TB; };

  gemm_tn_copy<kGemmBig, 8>(a.a, a.a_bytes, a.lda, a.K, 0, ca, stage_a(0), w);
  gemm_tn_copy<kGemmBig, 8>(a.b, a.b_bytes, a.ldb, a.K, 0, cb, stage_b(0), w);
  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{};

  for (int kt = 0; kt < nk; ++kt) {
    wait_vmcnt<0>();
    wg_barrier();
    if (kt + 1 < nk) {
      gemm_tn_copy<kGemmBig, 8>(a.a, a.a_bytes, a.lda, a.K, (kt + 1) * kGemmKT, ca, stage_a((kt + 1) & 1), w);
      gemm_tn_copy<kGemmBig, 8>(a.b, a.b_bytes, a.ldb, a.K, (kt + 1) * kGemmKT, cb, stage_b((kt + 1) & 1), w);
    }
    const MLA_LDS char* ta = stage_a(kt & 1);
    const MLA_LDS char* tb = stage_b(kt & 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 fa[8], fb[4];
#pragma unroll
      for (int t = 0; t < 8; ++t) fa[t] = gemm_tn_operand<kGemmBig>(ta, ks, 128 * wm + 16 * t, l16, kq);
#pragma unroll
      for (int t = 0; t < 4; ++t) fb[t] = gemm_tn_operand<kGemmBig>(tb, ks, 64 * wn + 16 * t, l16, kq);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(fa[i], fb[j], acc[i][j]);
    }
  }
  // C fragment (i, j): rows m0 + 128 wm + 16 i + 4 kq + e, column n0 + 64 wn + 16 j + l16
  float* C = a.c + (size_t)blockIdx.y * a.bsc;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 64 * wn + 16 * j + l16;
      if (n >= a.N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 128 * wm + 16 * i + 4 * kq + e;
        if (m < a.M) C[(size_t)m * a.N + n] = acc[i][j][e];
      }
    }
}

}  // namespace mla
