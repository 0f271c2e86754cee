// chunk_kda on gfx950: the KDA recurrence (page "符号表", section KDA 变量:
// per key channel log-space decay g, write strength beta, delta-rule
// residual r = v - k^T S_dec, write a = beta k, read-out o = q^T S; section
// Einsum 速查 for the three contractions; the summary list on the same page:
// the chunked form, a lower-triangular solve inside each chunk and the state
// carried between chunks, equals the step-by-step recurrence).
//
// Chunked form used here (C = 64 positions per chunk, state S_prev [K, V] at
// the chunk start, Gam_i = sum_{u<=i} g_u inside the chunk, a_j = beta_j k_j):
//   A_ij  = sum_c k_i[c] a_j[c] e^{Gam_i[c] - Gam_j[c]}       (j < i)
//   Bm_ij = sum_c q_i[c] a_j[c] e^{Gam_i[c] - Gam_j[c]}       (j <= i)
//   Tm = (I + A)^{-1},  W = Tm (k * e^Gam),  U = Tm v
//   R = U - W S_prev                      (the residuals r_i of the chunk)
//   O = (q * e^Gam) S_prev + Bm R         (the read-outs o_i)
//   S_next = e^{Gam_63} * S_prev + A_hat^T R,  A_hat_j = a_j * e^{Gam_63 - Gam_j}
//
// Two kernels:
//  * kda_intra, one workgroup per (batch, value head, chunk), fully parallel:
//    Gam, A and Bm (MFMA), the triangular solve (fp32, one wave), W and U
//    (MFMA).  It writes the per-chunk operands of the recurrence into a
//    workspace slot, each already in the row pitch the second kernel's LDS
//    reads want, so that kernel copies them with plain LDS-DMA.
//  * kda_state, one workgroup per (batch, value head, block of VB value
//    columns), walks the chunks in order with S (fp32) in registers: the
//    columns of S are independent, so a head's value columns split across
//    workgroups.  Each chunk's operands are double-buffered in LDS.
//
// e^{Gam_i - Gam_j} is never formed as e^{Gam_i} e^{-Gam_j} over the whole
// chunk (that overflows).  For A and Bm, row i of 16-row block I is scaled by
// e^{Gam_i - Gam_{16I}}, row j of block J by e^{Gam_{16J+15} - Gam_j} (both at
// most 1 for g <= 0) and the pair (I, J) by the per-channel factor
// F_IJ = e^{Gam_{16I} - Gam_{16J+15}}: at most 1 for J < I, and for J = I at
// most e^{15 |g|max}, which stays inside fp32 / bf16 range while every g is
// at least -5.9 (the pages' gate keeps g >= -5).
#pragma once

#include "common.h"

namespace kda {

using mla::bf16;
using mla::bf16x4;
using mla::bf16x8;
using mla::f32x4;
using mla::u32x4;

constexpr int kC = 64;  // chunk length

struct KdaArgs {
  const bf16* q;       // [B, T, H, K]
  const bf16* k;       // [B, T, H, K]
  const bf16* v;       // [B, T, HV, V]
  const float* g;      // [B, T, HV, K] log-space decay
  const float* beta;   // [B, T, HV]
  const float* s0;     // [B, HV, K, V] or null (zero state)
  bf16* o;             // [B, T, HV, V]
  float* s_out;        // [B, HV, K, V] or null
  char* ws;            // [B * HV * NC] slots of KdaDims::SLOT bytes
  int B, T, H, G, HV, NC;
  int xcd_map;         // kda_state: 1 = keep a head's value blocks on one XCD
};

__host__ __device__ constexpr int round_up(int x, int m) { return (x + m - 1) / m * m; }

template <int DK, int DV>
struct KdaDims {
  static constexpr int DKP = DK < 32 ? 32 : DK;  // channels padded to the MFMA k-step
  static constexpr int WP = DKP + 8;             // pitch (elements) of the W and q*e^Gam images
  static constexpr int TP = 72;                  // pitch of 64-wide rows (A_hat^T, Bm, U^T)
  static constexpr int W_BYTES = kC * WP * 2;
  static constexpr int AT_BYTES = DKP * TP * 2;
  static constexpr int B_BYTES = kC * TP * 2;
  static constexpr int UT_BYTES = DV * TP * 2;
  static constexpr int G_BYTES = DKP * 4;
  static constexpr int OFF_W = 0;
  static constexpr int OFF_Q = OFF_W + W_BYTES;
  static constexpr int OFF_AT = OFF_Q + W_BYTES;
  static constexpr int OFF_B = OFF_AT + AT_BYTES;
  static constexpr int OFF_UT = OFF_B + B_BYTES;
  static constexpr int OFF_G = OFF_UT + UT_BYTES;
  static constexpr int SLOT = round_up(OFF_G + G_BYTES, 256);
  static_assert(DK % 16 == 0 && DV % 16 == 0 && DK <= 128 && DV <= 128, "head widths");
  static_assert(W_BYTES % 16 == 0 && AT_BYTES % 16 == 0 && UT_BYTES % 16 == 0, "16-byte images");
};

__device__ __forceinline__ float exp_(float x) { return mla::fast_exp2(x * mla::kLog2e); }

__device__ __forceinline__ bf16x8 lds8(const MLA_LDS char* base, int byte_off) {
  return *(const MLA_LDS bf16x8*)(base + byte_off);
}

// ------------------------------------------------------------------ intra
template <int DK, int DV>
struct IntraLds {
  using D = KdaDims<DK, DV>;
  static constexpr int X_BYTES = kC * D::WP * 2;                   // one [64][WP] bf16 operand
  static constexpr int A_PITCH = 68;                               // fp32 A rows, 16-byte aligned
  static constexpr int RX = 2 * X_BYTES > kC * A_PITCH * 4 ? 2 * X_BYTES : kC * A_PITCH * 4;
  static constexpr int RY = X_BYTES > kC * D::TP * 2 ? X_BYTES : kC * D::TP * 2;
  static constexpr int OFF_XK = 0, OFF_XQ = X_BYTES, OFF_A = 0;    // A replaces XK / XQ after use
  static constexpr int OFF_Y = RX, OFF_T = RX;                     // Tm replaces Y after use
  static constexpr int OFF_F = RX + RY;
  static constexpr int OFF_KT = OFF_F + 10 * D::DKP * 4;
  static constexpr int OFF_VT = OFF_KT + D::DKP * D::TP * 2;
  static constexpr int OFF_BETA = OFF_VT + DV * D::TP * 2;
  static constexpr int BYTES = OFF_BETA + kC * 4;
};

// One workgroup (4 waves) per (batch, value head, chunk).
template <int DK, int DV>
__global__ void __launch_bounds__(256) kda_intra(KdaArgs a) {
  using D = KdaDims<DK, DV>;
  using L = IntraLds<DK, DV>;
  constexpr int DKP = D::DKP, WP = D::WP, TP = D::TP;
  __shared__ __attribute__((aligned(16))) char smem_raw[L::BYTES];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;
  bf16* sXK = (bf16*)(smem_raw + L::OFF_XK);
  bf16* sXQ = (bf16*)(smem_raw + L::OFF_XQ);
  bf16* sY = (bf16*)(smem_raw + L::OFF_Y);
  float* sF = (float*)(smem_raw + L::OFF_F);
  bf16* sKt = (bf16*)(smem_raw + L::OFF_KT);
  bf16* sVt = (bf16*)(smem_raw + L::OFF_VT);
  float* sBeta = (float*)(smem_raw + L::OFF_BETA);
  float* sA = (float*)(smem_raw + L::OFF_A);
  bf16* sT = (bf16*)(smem_raw + L::OFF_T);

  const int slot = blockIdx.x;
  const int ci = slot % a.NC, bh = slot / a.NC;
  const int hv = bh % a.HV, b = bh / a.HV, h = hv / a.G;
  const int t0 = ci * kC;
  const int nvalid = min(kC, a.T - t0);
  char* out = a.ws + (size_t)slot * D::SLOT;
  bf16* Qimg = (bf16*)(out + D::OFF_Q);
  bf16* Wimg = (bf16*)(out + D::OFF_W);
  bf16* Atimg = (bf16*)(out + D::OFF_AT);
  bf16* Bimg = (bf16*)(out + D::OFF_B);
  bf16* Utimg = (bf16*)(out + D::OFF_UT);
  float* Gimg = (float*)(out + D::OFF_G);
  const int tid = threadIdx.x;

  if (tid < kC) sBeta[tid] = tid < nvalid ? a.beta[((size_t)b * a.T + t0 + tid) * a.HV + hv] : 0.0f;
  __syncthreads();

  // ---- phase 1: one thread per key channel (Gam down the chunk, every
  // per-element scaling), one per value channel (V^T)
  if (tid < DKP) {
    const int ch = tid;
    const bool live = ch < DK;
    float gam[kC];
    float run = 0.0f;
#pragma unroll
    for (int i = 0; i < kC; ++i) {
      float gi = 0.0f;
      if (live && i < nvalid) gi = a.g[(((size_t)b * a.T + t0 + i) * a.HV + hv) * DK + ch];
      run += gi;
      gam[i] = run;
    }
    const float gl = gam[kC - 1];
    Gimg[ch] = live ? exp_(gl) : 1.0f;
#pragma unroll
    for (int i8 = 0; i8 < kC / 8; ++i8) {
      bf16x8 kt8, at8;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = 8 * i8 + u;
        float kk = 0.0f, qq = 0.0f;
        if (live && i < nvalid) {
          const size_t idx = (((size_t)b * a.T + t0 + i) * a.H + h) * DK + ch;
          kk = (float)a.k[idx];
          qq = (float)a.q[idx];
        }
        const float bi = sBeta[i];
        const float e = exp_(gam[i]);
        kt8[u] = (bf16)(kk * e);
        at8[u] = (bf16)(bi * kk * exp_(gl - gam[i]));
        const int r0 = 16 * (i / 16);
        const float eb = exp_(gam[i] - gam[r0]);
        sXK[i * WP + ch] = (bf16)(kk * eb);
        sXQ[i * WP + ch] = (bf16)(qq * eb);
        sY[i * WP + ch] = (bf16)(bi * kk * exp_(gam[r0 + 15] - gam[i]));
        Qimg[i * WP + ch] = (bf16)(qq * e);
      }
      *(bf16x8*)&sKt[ch * TP + 8 * i8] = kt8;
      *(bf16x8*)&Atimg[ch * TP + 8 * i8] = at8;
    }
    int p = 0;
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int J = 0; J <= I; ++J) sF[(p++) * DKP + ch] = exp_(gam[16 * I] - gam[16 * J + 15]);
  } else if (tid < DKP + DV) {
    const int ch = tid - DKP;
#pragma unroll
    for (int i8 = 0; i8 < kC / 8; ++i8) {
      bf16x8 v8;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = 8 * i8 + u;
        v8[u] = i < nvalid ? a.v[(((size_t)b * a.T + t0 + i) * a.HV + hv) * DV + ch] : (bf16)0.0f;
      }
      *(bf16x8*)&sVt[ch * TP + 8 * i8] = v8;
    }
  }
  __syncthreads();

  // ---- phase 2: A and Bm, wave w owns block row I = w (blocks J <= I)
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, kq = lane >> 4;
  f32x4 accA[4], accB[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) accA[J] = accB[J] = f32x4{};
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    if (J > w) continue;
    const int pair = w * (w + 1) / 2 + J;
#pragma unroll
    for (int ks = 0; ks < DKP / 32; ++ks) {
      const int c0 = 32 * ks + 8 * kq;
      const bf16x8 xk = lds8(smem, L::OFF_XK + ((16 * w + l16) * WP + c0) * 2);
      const bf16x8 xq = lds8(smem, L::OFF_XQ + ((16 * w + l16) * WP + c0) * 2);
      const bf16x8 y = lds8(smem, L::OFF_Y + ((16 * J + l16) * WP + c0) * 2);
      const f32x4 f0 = *(const f32x4*)&sF[pair * DKP + c0];
      const f32x4 f1 = *(const f32x4*)&sF[pair * DKP + c0 + 4];
      bf16x8 xk2, xq2;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float f = u < 4 ? f0[u] : f1[u - 4];
        xk2[u] = (bf16)((float)xk[u] * f);
        xq2[u] = (bf16)((float)xq[u] * f);
      }
      accA[J] = mla::mfma16(xk2, y, accA[J]);
      accB[J] = mla::mfma16(xq2, y, accB[J]);
    }
  }
  // Bm image (rows i = 16 w + 4 kq + e, column j = 16 J + l16), zero above the diagonal
#pragma unroll
  for (int J = 0; J < 4; ++J)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * w + 4 * kq + e, j = 16 * J + l16;
      Bimg[i * TP + j] = (bf16)(j <= i ? accB[J][e] : 0.0f);
    }
  __syncthreads();  // every wave is done with XK / XQ / Y
#pragma unroll
  for (int J = 0; J < 4; ++J)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * w + 4 * kq + e, j = 16 * J + l16;
      sA[i * L::A_PITCH + j] = j < i ? accA[J][e] : 0.0f;
    }
  __syncthreads();

  // ---- phase 3: Tm = (I + A)^{-1}, lane c solves column c by forward substitution
  if (w == 0) {
    float x[kC];
#pragma unroll
    for (int i = 0; i < kC; ++i) {
      float acc = (i == lane) ? 1.0f : 0.0f;
#pragma unroll
      for (int j4 = 0; j4 < i / 4; ++j4) {
        const f32x4 av = *(const f32x4*)&sA[i * L::A_PITCH + 4 * j4];
        acc -= av[0] * x[4 * j4] + av[1] * x[4 * j4 + 1] + av[2] * x[4 * j4 + 2] + av[3] * x[4 * j4 + 3];
      }
#pragma unroll
      for (int j = 4 * (i / 4); j < i; ++j) acc -= sA[i * L::A_PITCH + j] * x[j];
      x[i] = acc;
    }
#pragma unroll
    for (int i = 0; i < kC; ++i) sT[i * TP + lane] = (bf16)x[i];
  }
  __syncthreads();

  // ---- phase 4: W^T = (k e^Gam)^T Tm^T (tiles: 16 channels x 16 rows) and
  // U = Tm V (tiles: 16 rows x 16 value channels)
  constexpr int NWT = (DKP / 16) * 4, NUT = 4 * (DV / 16);
  for (int tile = w; tile < NWT + NUT; tile += 4) {
    f32x4 acc = f32x4{};
    if (tile < NWT) {
      const int C = tile / 4, I = tile % 4;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int j0 = 32 * ks + 8 * kq;
        acc = mla::mfma16(lds8(smem, L::OFF_KT + ((16 * C + l16) * TP + j0) * 2),
                          lds8(smem, L::OFF_T + ((16 * I + l16) * TP + j0) * 2), acc);
      }
      // rows channel 16 C + 4 kq + e, column i = 16 I + l16: W[i][c .. c+3]
      bf16x4 w4;
#pragma unroll
      for (int e = 0; e < 4; ++e) w4[e] = (bf16)acc[e];
      *(bf16x4*)&Wimg[(16 * I + l16) * WP + 16 * C + 4 * kq] = w4;
    } else {
      const int t = tile - NWT, I = t % 4, V = t / 4;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int j0 = 32 * ks + 8 * kq;
        acc = mla::mfma16(lds8(smem, L::OFF_T + ((16 * I + l16) * TP + j0) * 2),
                          lds8(smem, L::OFF_VT + ((16 * V + l16) * TP + j0) * 2), acc);
      }
      // rows i = 16 I + 4 kq + e, column v = 16 V + l16: U^T[v][i .. i+3]
      bf16x4 u4;
#pragma unroll
      for (int e = 0; e < 4; ++e) u4[e] = (bf16)acc[e];
      *(bf16x4*)&Utimg[(16 * V + l16) * TP + 16 * I + 4 * kq] = u4;
    }
  }
}

// ------------------------------------------------------------------ state
// Copies NB bytes (a multiple of 16) from global src into LDS dst: 1 KiB
// pieces, piece p issued by wave p % 4, the lanes of a last partial piece
// past NB masked off (so nothing past dst + NB is written).
template <int NB>
__device__ __forceinline__ void copy_image(const char* src, MLA_LDS char* dst, int w, int lane) {
  static_assert(NB % 16 == 0, "16-byte pieces");
  constexpr int PIECES = (NB + 1023) / 1024;
  const u32x4 rs = mla::make_rsrc(src, (unsigned)NB);
#pragma unroll
  for (int p = 0; p < PIECES; ++p) {
    if (p % 4 != w) continue;
    if (p * 1024 + 16 * lane < NB) mla::buf2lds16(rs, (unsigned)(p * 1024 + 16 * lane), dst + p * 1024);
  }
}

template <int DK, int DV, int VB>
struct StateLds {
  using D = KdaDims<DK, DV>;
  static constexpr int S_W = 0;
  static constexpr int S_Q = S_W + D::W_BYTES;
  static constexpr int S_AT = S_Q + D::W_BYTES;
  static constexpr int S_B = S_AT + D::AT_BYTES;
  static constexpr int S_UT = S_B + D::B_BYTES;
  static constexpr int UT_SLICE = VB * D::TP * 2;
  static constexpr int S_G = S_UT + UT_SLICE;
  static constexpr int STAGE = round_up(S_G + D::G_BYTES, 16);
  static constexpr int OFF_ST = 2 * STAGE;                      // S^T bf16 [VB][WP]
  static constexpr int OFF_RT = OFF_ST + VB * D::WP * 2;        // R^T bf16 [VB][TP]
  static constexpr int BYTES = OFF_RT + VB * D::TP * 2;
};

// One workgroup (4 waves) per (batch, value head, VB value columns); wave w
// owns rows 16 w .. of R and O and channel tiles w, w+4, ... of S.
template <int DK, int DV, int VB>
__global__ void __launch_bounds__(256) kda_state(KdaArgs a) {
  using D = KdaDims<DK, DV>;
  using L = StateLds<DK, DV, VB>;
  constexpr int DKP = D::DKP, WP = D::WP, TP = D::TP;
  constexpr int NVB = DV / VB, NVT = VB / 16, NCT = DKP / 16, CPW = (NCT + 3) / 4;
  static_assert(DV % VB == 0 && VB % 16 == 0, "value blocks");
  __shared__ __attribute__((aligned(1024))) char smem_raw[L::BYTES];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;
  bf16* sSt = (bf16*)(smem_raw + L::OFF_ST);
  bf16* sRt = (bf16*)(smem_raw + L::OFF_RT);

  // a head's NVB value blocks on one XCD (workgroups are dealt to the 8 XCDs
  // round-robin) when the head count allows it
  const int id = blockIdx.x;
  int bh, vb;
  if (a.xcd_map) {
    vb = (id / 8) % NVB;
    bh = (id % 8) + 8 * (id / (8 * NVB));
  } else {
    vb = id % NVB;
    bh = id / NVB;
  }
  const int hv = bh % a.HV, b = bh / a.HV;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, kq = lane >> 4;
  const int v0 = vb * VB;

  auto issue = [&](int ci, int st) {
    const char* slot = a.ws + ((size_t)bh * a.NC + ci) * D::SLOT;
    MLA_LDS char* dst = smem + st * L::STAGE;
    copy_image<D::W_BYTES>(slot + D::OFF_W, dst + L::S_W, w, lane);
    copy_image<D::W_BYTES>(slot + D::OFF_Q, dst + L::S_Q, w, lane);
    copy_image<D::AT_BYTES>(slot + D::OFF_AT, dst + L::S_AT, w, lane);
    copy_image<D::B_BYTES>(slot + D::OFF_B, dst + L::S_B, w, lane);
    copy_image<L::UT_SLICE>(slot + D::OFF_UT + v0 * TP * 2, dst + L::S_UT, w, lane);
    copy_image<D::G_BYTES>(slot + D::OFF_G, dst + L::S_G, w, lane);
  };
  issue(0, 0);

  // the state: fragment (m, V) holds channels 16 (w + 4 m) + 4 kq + e of value column 16 V + l16
  f32x4 S[CPW][NVT];
#pragma unroll
  for (int m = 0; m < CPW; ++m) {
    const int C = w + 4 * m;
#pragma unroll
    for (int V = 0; V < NVT; ++V) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 16 * C + 4 * kq + e;
        S[m][V][e] = (a.s0 && C < NCT && c < DK)
                         ? a.s0[(((size_t)b * a.HV + hv) * DK + c) * DV + v0 + 16 * V + l16]
                         : 0.0f;
      }
      if (C < NCT) {
        bf16x4 s4;
#pragma unroll
        for (int e = 0; e < 4; ++e) s4[e] = (bf16)S[m][V][e];
        *(bf16x4*)&sSt[(16 * V + l16) * WP + 16 * C + 4 * kq] = s4;
      }
    }
  }

  for (int ci = 0; ci < a.NC; ++ci) {
    mla::wait_vmcnt<0>();
    mla::wait_lgkmcnt0();
    mla::wg_barrier();  // chunk ci staged, S^T of the previous chunk written, R^T free
    if (ci + 1 < a.NC) issue(ci + 1, (ci + 1) & 1);
    const int so = (ci & 1) * L::STAGE;

    // R = U - W S and P = (q e^Gam) S: rows 16 w + 4 kq + e, value column 16 V + l16
    f32x4 accR[NVT], accP[NVT];
#pragma unroll
    for (int V = 0; V < NVT; ++V) accR[V] = accP[V] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < DKP / 32; ++ks) {
      const int c0 = 32 * ks + 8 * kq;
      const bf16x8 aw = lds8(smem, so + L::S_W + ((16 * w + l16) * WP + c0) * 2);
      const bf16x8 aq = lds8(smem, so + L::S_Q + ((16 * w + l16) * WP + c0) * 2);
#pragma unroll
      for (int V = 0; V < NVT; ++V) {
        const bf16x8 bs = lds8(smem, L::OFF_ST + ((16 * V + l16) * WP + c0) * 2);
        accR[V] = mla::mfma16(aw, bs, accR[V]);
        accP[V] = mla::mfma16(aq, bs, accP[V]);
      }
    }
#pragma unroll
    for (int V = 0; V < NVT; ++V) {
      const bf16x4 u4 = *(const MLA_LDS bf16x4*)(smem + so + L::S_UT + ((16 * V + l16) * TP + 16 * w + 4 * kq) * 2);
      bf16x4 r4;
#pragma unroll
      for (int e = 0; e < 4; ++e) r4[e] = (bf16)((float)u4[e] - accR[V][e]);
      *(bf16x4*)&sRt[(16 * V + l16) * TP + 16 * w + 4 * kq] = r4;
    }
    mla::wait_lgkmcnt0();
    mla::wg_barrier();  // R^T complete; every wave is done reading S^T

    // O = P + Bm R
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int j0 = 32 * ks + 8 * kq;
      const bf16x8 ab = lds8(smem, so + L::S_B + ((16 * w + l16) * TP + j0) * 2);
#pragma unroll
      for (int V = 0; V < NVT; ++V)
        accP[V] = mla::mfma16(ab, lds8(smem, L::OFF_RT + ((16 * V + l16) * TP + j0) * 2), accP[V]);
    }
    const int t0 = ci * kC;
#pragma unroll
    for (int V = 0; V < NVT; ++V)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + 16 * w + 4 * kq + e;
        if (t < a.T) a.o[(((size_t)b * a.T + t) * a.HV + hv) * DV + v0 + 16 * V + l16] = (bf16)accP[V][e];
      }

    // S = e^{Gam_63} S + A_hat^T R
#pragma unroll
    for (int m = 0; m < CPW; ++m) {
      const int C = w + 4 * m;
      if (C >= NCT) continue;
      const f32x4 gc = *(const MLA_LDS f32x4*)(smem + so + L::S_G + (16 * C + 4 * kq) * 4);
#pragma unroll
      for (int V = 0; V < NVT; ++V)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[m][V][e] *= gc[e];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int j0 = 32 * ks + 8 * kq;
        const bf16x8 aa = lds8(smem, so + L::S_AT + ((16 * C + l16) * TP + j0) * 2);
#pragma unroll
        for (int V = 0; V < NVT; ++V)
          S[m][V] = mla::mfma16(aa, lds8(smem, L::OFF_RT + ((16 * V + l16) * TP + j0) * 2), S[m][V]);
      }
#pragma unroll
      for (int V = 0; V < NVT; ++V) {
        bf16x4 s4;
#pragma unroll
        for (int e = 0; e < 4; ++e) s4[e] = (bf16)S[m][V][e];
        *(bf16x4*)&sSt[(16 * V + l16) * WP + 16 * C + 4 * kq] = s4;
      }
    }
  }

  if (a.s_out) {
#pragma unroll
    for (int m = 0; m < CPW; ++m) {
      const int C = w + 4 * m;
      if (C >= NCT) continue;
#pragma unroll
      for (int V = 0; V < NVT; ++V)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = 16 * C + 4 * kq + e;
          if (c < DK) a.s_out[(((size_t)b * a.HV + hv) * DK + c) * DV + v0 + 16 * V + l16] = S[m][V][e];
        }
    }
  }
}

}  // namespace kda
