// Pieces of the full Gated MLA forward around the absorbed core (page "Gated
// MLA（矩阵吸收版）", section 低秩压缩 for c = RMSNorm(W_down x) and section
// 完整计算流（四步） step 1 for the query low-rank path): the row RMSNorm of the
// two down-projections.  The projections themselves are mla_gemm_nt.
#pragma once

#include "common.h"

namespace mla {

struct RmsNormArgs {
  const bf16* x;     // [rows, n]
  bf16* y;           // [rows, n] the normalised rows (may be x itself)
  const bf16* gain;  // [n]
  float* rstd;       // [rows] 1 / sqrt(mean(x^2) + eps), kept for the backward (null: not kept)
  int rows, n;
  float eps;         // added to the mean square inside the square root
};

// One wave per row: y = x / sqrt(mean(x^2) + eps) * gain, fp32 arithmetic.
// n is a multiple of 8 and at most 64 * 8 * kMaxChunks.
constexpr int kNormMaxChunks = 4;  // n <= 2048

__global__ void __launch_bounds__(256) mla_rmsnorm_rows(RmsNormArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= a.rows) return;
  const bf16* xr = a.x + (size_t)row * a.n;
  bf16* yr = a.y + (size_t)row * a.n;
  bf16x8 v[kNormMaxChunks];
  float ss = 0.0f;
#pragma unroll
  for (int u = 0; u < kNormMaxChunks; ++u) {
    const int j = 8 * (lane + 64 * u);
    v[u] = j < a.n ? *(const bf16x8*)(xr + j) : bf16x8{};
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += (float)v[u][e] * (float)v[u][e];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
  const float inv = 1.0f / __builtin_sqrtf(ss / (float)a.n + a.eps);
  if (a.rstd && lane == 0) a.rstd[row] = inv;
#pragma unroll
  for (int u = 0; u < kNormMaxChunks; ++u) {
    const int j = 8 * (lane + 64 * u);
    if (j < a.n) {
      const bf16x8 g = *(const bf16x8*)(a.gain + j);
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (bf16)((float)v[u][e] * inv * (float)g[e]);
      *(bf16x8*)(yr + j) = o;
    }
  }
}

}  // namespace mla
