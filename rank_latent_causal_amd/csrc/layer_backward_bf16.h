// Pieces of the backward of the full Gated MLA layer (page "Gated MLA（矩阵吸收
// 版）", section 低秩压缩 for the latent norm and section 完整计算流（四步）
// step 1 for the query norm, differentiated by the chain rule): the RMSNorm
// backward with its gain gradient, the column sums that finish the gain
// gradient, and a strided transpose that lays weights out for the
// input-gradient products (run as mla_gemm_nt).
#pragma once

#include "common.h"
#include "forward_bf16.h"

namespace mla {

struct RmsNormBwdArgs {
  const bf16* du;     // [rows, n] gradient of the norm's output, rows ld_du apart
  const bf16* v;      // [rows, n] the norm's input
  const float* rstd;  // [rows] 1 / sqrt(mean(v^2) + eps) of the forward
  const bf16* gain;   // [n]
  bf16* dv;           // [rows, n] gradient of the norm's input, rows ld_dv apart
  float* part;        // [gridDim.x, n] per-workgroup partial sums of du * v * rstd
  int rows, n, ld_du, ld_dv;
};

// For u = g * v * rstd, with nrm = v * rstd:
//   dv = (du * g - nrm * mean(du * g * nrm)) * rstd,   dg = sum over rows of du * nrm.
// Each wave takes rows w, w + (waves in the grid), ... (one row per pass,
// eight values per lane and chunk); the gain gradient accumulates in
// registers, then across the four waves in LDS into one partial row per
// workgroup.  n is a multiple of 8 and at most 64 * 8 * kNormMaxChunks.
__global__ void __launch_bounds__(256) mla_rmsnorm_backward(RmsNormBwdArgs a) {
  constexpr int U = kNormMaxChunks;
  __shared__ float red[4][64 * 8 * U];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float g[U][8], acc[U][8];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = 8 * (lane + 64 * u);
    const bf16x8 gv = j < a.n ? *(const bf16x8*)(a.gain + j) : bf16x8{};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      g[u][e] = (float)gv[e];
      acc[u][e] = 0.0f;
    }
  }
  const float inv_n = 1.0f / (float)a.n;
  for (int row = blockIdx.x * 4 + w; row < a.rows; row += gridDim.x * 4) {
    const bf16* dur = a.du + (size_t)row * a.ld_du;
    const bf16* vr = a.v + (size_t)row * a.n;
    const float rs = a.rstd[row];
    float du[U][8], nrm[U][8];
    float dot = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = 8 * (lane + 64 * u);
      const bf16x8 dv8 = j < a.n ? *(const bf16x8*)(dur + j) : bf16x8{};
      const bf16x8 vv8 = j < a.n ? *(const bf16x8*)(vr + j) : bf16x8{};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        du[u][e] = (float)dv8[e];
        nrm[u][e] = (float)vv8[e] * rs;
        dot += du[u][e] * g[u][e] * nrm[u][e];
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) dot += __shfl_xor(dot, o, 64);
    dot *= inv_n;
    bf16* dvr = a.dv + (size_t)row * a.ld_dv;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = 8 * (lane + 64 * u);
      if (j < a.n) {
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o[e] = (bf16)((du[u][e] * g[u][e] - nrm[u][e] * dot) * rs);
          acc[u][e] += du[u][e] * nrm[u][e];
        }
        *(bf16x8*)(dvr + j) = o;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = 8 * (lane + 64 * u);
    if (j < a.n)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[w][j + e] = acc[u][e];
  }
  __syncthreads();
  for (int j = threadIdx.x; j < a.n; j += 256)
    a.part[(size_t)blockIdx.x * a.n + j] = red[0][j] + red[1][j] + red[2][j] + red[3][j];
}

// out[j] = sum over p < nparts of part[p, j] (fp32, fixed order)
__global__ void __launch_bounds__(256) mla_colsum_f32(const float* __restrict__ part, int nparts, int n,
                                                      float* __restrict__ out) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  float s = 0.0f;
  for (int p = 0; p < nparts; ++p) s += part[(size_t)p * n + j];
  out[j] = s;
}

// dst[j, i] = src[i, j] for src [rows, cols] (dense) and dst rows ld_dst
// apart: one 32 x 32 tile per workgroup through LDS.
__global__ void __launch_bounds__(256) mla_transpose_into(const bf16* __restrict__ src, int rows, int cols,
                                                          bf16* __restrict__ dst, long long ld_dst) {
  __shared__ bf16 tile[32][33];
  const int j0 = blockIdx.x * 32, i0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = i0 + ty + 8 * k, j = j0 + tx;
    if (i < rows && j < cols) tile[ty + 8 * k][tx] = src[(size_t)i * cols + j];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int j = j0 + ty + 8 * k, i = i0 + tx;
    if (i < rows && j < cols) dst[(size_t)j * ld_dst + i] = tile[tx][ty + 8 * k];
  }
}

}  // namespace mla
