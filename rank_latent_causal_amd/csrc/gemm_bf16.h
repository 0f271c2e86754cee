// bf16 GEMM for the projections around the absorbed core (page "Gated MLA
// （矩阵吸收版）", section 完整计算流（四步）: the query low-rank path of step 1,
// the latent down-projection of section 低秩压缩, the gate and the output
// projection of step 4).  Every projection is a linear layer
//
//   Y[m, n] = sum_k X[m, k] * W[n, k]        X [M, K], W [N, K], Y [M, N]
//
// (row-major, K contiguous in both operands, the weight laid out as
// out_features x in_features), bf16 storage with fp32 accumulation.
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
  const bf16* x;  // [M, K]
  const bf16* w;  // [N, K]
  bf16* y;        // [M, N]
  int M, N, K;    // K % 64 == 0
  int tiles_n;    // ceil(N / 128)
};

constexpr int kGemmTile = 128;
constexpr int kGemmKT = 64;
constexpr int kGemmTileBytes = kGemmTile * kGemmKT * 2;  // 16 KiB per operand per stage

__device__ __forceinline__ int gemm_chunk(int s, int c) { return c ^ ((s >> 1) & 7); }

// Copies rows [row0, row0 + 128) x k [k0, k0 + 64) of a K-contiguous
// operand into a swizzled LDS tile.  Copy i (1 KiB = 8 rows) is issued by
// wave i % 4; lane l of a copy fills LDS bytes 16 l .. of it, which is row
// 8 i + l / 8, physical chunk l % 8.
__device__ __forceinline__ void gemm_copy(const bf16* __restrict__ base, int rows_total, int row0, int K,
                                          int k0, MLA_LDS char* tile, int w) {
  unsigned ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  int rows = rows_total - row0;
  rows = rows > kGemmTile ? kGemmTile : rows;
  const u32x4 rs = make_rsrc(base + (size_t)row0 * K, (unsigned)((size_t)(rows > 0 ? rows : 0) * K * 2));
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int i = w + 4 * c;  // copy index 0..15
    const int s = 8 * i + (int)(ln >> 3);
    const int logical = gemm_chunk(s, (int)(ln & 7));
    const unsigned voff = (unsigned)((s * K + k0 + 8 * logical) * 2);
    buf2lds16(rs, voff, tile + i * 1024);
  }
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
mla_gemm_nt(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * 2 * kGemmTileBytes];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;  // [stage][W tile, X tile]

  const int tn = blockIdx.x % a.tiles_n, tm = blockIdx.x / a.tiles_n;
  const int n0 = tn * kGemmTile, m0 = tm * kGemmTile;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, kq = lane >> 4;
  const int wn = w & 1, wm = w >> 1;  // this wave's 64 x 64 block
  const int nk = a.K / kGemmKT;

  auto stage_w = [&](int st) { return smem + st * 2 * kGemmTileBytes; };
  auto stage_x = [&](int st) { return smem + st * 2 * kGemmTileBytes + kGemmTileBytes; };

  gemm_copy(a.w, a.N, n0, a.K, 0, stage_w(0), w);
  gemm_copy(a.x, a.M, m0, a.K, 0, stage_x(0), w);

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
      gemm_copy(a.w, a.N, n0, a.K, (kt + 1) * kGemmKT, stage_w((kt + 1) & 1), w);
      gemm_copy(a.x, a.M, m0, a.K, (kt + 1) * kGemmKT, stage_x((kt + 1) & 1), w);
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
      for (int e = 0; e < 4; ++e) v[e] = (bf16)acc[i][j][e];
      bf16* dst = a.y + (size_t)m * a.N + n;
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

}  // namespace mla
