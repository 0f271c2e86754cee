// fp32 kernels for the absorbed Gated MLA layer (the toy-size precision path).
//
// One wave evaluates one (query row, head): the latent dimension r is spread
// over the 64 lanes (r <= 1024, 16 values per lane), each key's score is a
// wave reduction, the softmax is online in fp32, and the W_UV^T product is a
// wave reduction per output column.  Same definition as the bf16 path
// (page "Gated MLA（矩阵吸收版）", section 完整计算流（四步） steps 2-4) with no
// narrowing of any intermediate.
#pragma once

#include "common.h"

namespace mla {

struct F32Args {
  const float* q;      // prefill [B, T, H, DQ]   decode [B, H, DQ]
  const float* c;      // prefill [B, S, R]       decode [N, R]
  const int* cu;       // decode only: [B + 1]
  const float* wuk;    // [H, DQ, R]
  const float* wuv;    // [H, DV, R]
  const float* gate;   // [rows, H*DV]
  float* out;          // [rows, H*DV]
  int B, T, H, DQ, DV, R;
  int S;               // prefill: latent rows per sequence (S >= T; the T queries are the last T positions)
  long long N;         // decode: cache rows
  float scale;
  int decode;
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// grid: (rows, H); block: 64 threads.  rows = B*T (prefill) or B (decode).
__global__ void __launch_bounds__(64) mla_f32_kernel(F32Args a) {
  constexpr int MAXJ = 16;  // r <= 64 * 16
  const int row = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int R = a.R, DQ = a.DQ, DV = a.DV, H = a.H;
  long long key_lo, key_hi;
  const float* keys;
  if (a.decode) {
    key_lo = a.cu[row];
    key_hi = a.cu[row + 1];
    key_lo = key_lo < a.N ? key_lo : a.N;
    key_hi = key_hi < a.N ? key_hi : a.N;
    keys = a.c;
  } else {
    const int b = row / a.T, t = row % a.T;
    key_lo = 0;
    key_hi = (a.S - a.T) + t + 1;
    keys = a.c + (size_t)b * a.S * R;
  }
  const float* qrow = a.q + ((size_t)row * H + h) * DQ;
  const float* wk = a.wuk + (size_t)h * DQ * R;

  // q_abs (this lane's columns j = lane + 64 u)
  float qa[MAXJ];
#pragma unroll
  for (int u = 0; u < MAXJ; ++u) {
    const int j = lane + 64 * u;
    float s = 0.0f;
    if (j < R)
      for (int d = 0; d < DQ; ++d) s = fmaf(qrow[d], wk[(size_t)d * R + j], s);
    qa[u] = s;
  }

  float m = -INFINITY, l = 0.0f;
  float ol[MAXJ];
#pragma unroll
  for (int u = 0; u < MAXJ; ++u) ol[u] = 0.0f;
  for (long long s = key_lo; s < key_hi; ++s) {
    const float* cr = keys + (size_t)s * R;
    float part = 0.0f;
#pragma unroll
    for (int u = 0; u < MAXJ; ++u) {
      const int j = lane + 64 * u;
      if (j < R) part = fmaf(qa[u], cr[j], part);
    }
    const float sc = wave_sum(part) * a.scale;
    const float mn = fmaxf(m, sc);
    const float alpha = expf(m - mn);
    const float p = expf(sc - mn);
    l = l * alpha + p;
#pragma unroll
    for (int u = 0; u < MAXJ; ++u) {
      const int j = lane + 64 * u;
      ol[u] = ol[u] * alpha + (j < R ? p * cr[j] : 0.0f);
    }
    m = mn;
  }
  const float inv = 1.0f / l;
  const float* wv = a.wuv + (size_t)h * DV * R;
  const size_t orow = (size_t)row * H * DV + (size_t)h * DV;
  for (int v = 0; v < DV; ++v) {
    float part = 0.0f;
#pragma unroll
    for (int u = 0; u < MAXJ; ++u) {
      const int j = lane + 64 * u;
      if (j < R) part = fmaf(ol[u] * inv, wv[(size_t)v * R + j], part);
    }
    const float o = wave_sum(part);
    if (lane == 0) {
      const float gv = a.gate[orow + v];
      a.out[orow + v] = o / (1.0f + expf(-gv));
    }
  }
}

}  // namespace mla
