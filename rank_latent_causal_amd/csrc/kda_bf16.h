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
  static constexpr int X_BYTES = kC * D::DKP * 2;  // X_K / X_Q: [64][DKP] bf16, chunk-swizzled rows
  static constexpr int Y_BYTES = kC * D::WP * 2;   // Y: [64][WP] bf16
  static constexpr int A_PITCH = 68;               // fp32 A / Tm rows, 16-byte aligned
  static constexpr int A_BYTES = kC * A_PITCH * 4;
  static constexpr int P_BYTES = 4 * 16 * 16 * 4;  // one 16 x 16 fp32 product per wave
  static constexpr int T_BYTES = kC * D::TP * 2;   // bf16 Tm [64][TP]
  static constexpr int max2(int x, int y) { return x > y ? x : y; }
  // Region lifetimes (phases 0-4):
  //   R1: raw k -> X_K (0-2), A (3), K~^T (4, spilling into R2)
  //   R2: raw q -> X_Q (0-2), fp32 Tm (3)
  //   R3: raw decays (0-1a), Y and F (1b-2), the solve's products then bf16 Tm (3-4), V^T (4)
  static constexpr int R1 = max2(X_BYTES, A_BYTES), R2 = max2(X_BYTES, A_BYTES);
  static constexpr int OFF_R1 = 0, OFF_R2 = R1, OFF_R3 = R1 + R2;
  static constexpr int R3 = max2(max2(kC * D::DKP * 4, Y_BYTES + 10 * D::DKP * 4), max2(P_BYTES, T_BYTES) + DV * D::TP * 2);
  static constexpr int OFF_XK = OFF_R1, OFF_A = OFF_R1, OFF_KT = OFF_R1;
  static constexpr int OFF_XQ = OFF_R2, OFF_TF = OFF_R2;
  static constexpr int OFF_G = OFF_R3, OFF_Y = OFF_R3, OFF_F = OFF_R3 + Y_BYTES;
  static constexpr int OFF_P = OFF_R3, OFF_T = OFF_R3, OFF_VT = OFF_R3 + max2(P_BYTES, T_BYTES);
  static constexpr int OFF_BETA = OFF_R3 + R3;
  static constexpr int BYTES = OFF_BETA + kC * 4;
  static_assert(D::DKP * D::TP * 2 <= R1 + R2, "K~^T fits over A and Tm");
};

// X_K / X_Q rows are 2 DKP bytes, unpadded, so the LDS-DMA copy can fill
// whole rows; the 16-byte chunk L of row i sits at chunk L ^ xswz(i), which
// spreads the 16 consecutive rows of an MFMA operand read over all banks.
template <int DKP>
__device__ __forceinline__ int xswz(int i) {
  constexpr int CPR = DKP / 8, RPB = 256 / (2 * DKP);  // chunks per row, rows per 256 bytes
  return (i / RPB) % CPR;
}
template <int DKP>
__device__ __forceinline__ int xoff(int i, int ch) {  // byte offset of element (i, ch)
  return i * (2 * DKP) + ((((ch >> 3) ^ xswz<DKP>(i))) << 4) + (ch & 7) * 2;
}

// Workgroup barrier that orders LDS only: this wave's LDS accesses have
// completed, then s_barrier.  __syncthreads() would also wait for every
// global store still in flight (the images written to the workspace).
__device__ __forceinline__ void lds_barrier() {
  mla::wait_lgkmcnt0();
  mla::wg_barrier();
}

// Waves of kda_intra: 8 at K = 128 (four threads per key channel in the
// scaling phase, A and Bm on separate waves), 4 for the narrower heads.
template <int DK>
constexpr int intra_waves() { return DK >= 128 ? 8 : 4; }

// One workgroup per (batch, value head, chunk); two fit on a CU.
template <int DK, int DV>
__global__ void __launch_bounds__(64 * intra_waves<DK>()) kda_intra(KdaArgs a) {
  constexpr int NW = intra_waves<DK>(), NT = 64 * NW;
  using D = KdaDims<DK, DV>;
  using L = IntraLds<DK, DV>;
  constexpr int DKP = D::DKP, WP = D::WP, TP = D::TP, AP = L::A_PITCH;
  __shared__ __attribute__((aligned(16))) char smem_raw[L::BYTES];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;
  bf16* sY = (bf16*)(smem_raw + L::OFF_Y);
  float* sF = (float*)(smem_raw + L::OFF_F);
  float* sG = (float*)(smem_raw + L::OFF_G);
  float* sA = (float*)(smem_raw + L::OFF_A);
  float* sTf = (float*)(smem_raw + L::OFF_TF);
  bf16* sT = (bf16*)(smem_raw + L::OFF_T);
  bf16* sKt = (bf16*)(smem_raw + L::OFF_KT);
  bf16* sVt = (bf16*)(smem_raw + L::OFF_VT);
  float* sBeta = (float*)(smem_raw + L::OFF_BETA);

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
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l16 = lane & 15, kq = lane >> 4;

  // ---- phase 0: k and q rows (chunk-swizzled) and the decays go straight
  // from global memory into LDS with LDS-DMA copies (rows past the chunk's
  // end and channels past K read as zeros); v is loaded into registers and
  // written transposed once the solve is done
  constexpr int VCH = DV / 8, NV = kC * VCH, VPER = (NV + NT - 1) / NT;
  bf16x8 vreg[VPER];
  {
    constexpr int CPR = DKP / 8, RPK = 1024 / (2 * DKP);        // key rows per 1 KiB copy
    constexpr int GPR = DKP / 4, GRK = 1024 / (4 * DKP);        // decay chunks per row, rows per copy
    constexpr int NKC = kC / RPK, NGC = kC / GRK;               // copies per key tensor, for the decays
    const u32x4 rk = mla::make_rsrc(a.k + (size_t)b * a.T * a.H * DK, (unsigned)((size_t)a.T * a.H * DK * 2));
    const u32x4 rq = mla::make_rsrc(a.q + (size_t)b * a.T * a.H * DK, (unsigned)((size_t)a.T * a.H * DK * 2));
    const u32x4 rg = mla::make_rsrc(a.g + (size_t)b * a.T * a.HV * DK, (unsigned)((size_t)a.T * a.HV * DK * 4));
    for (int c = w; c < 2 * NKC + NGC; c += NW) {
      if (c < 2 * NKC) {
        const int cc = c % NKC, i = RPK * cc + lane / CPR;
        const int L = (lane % CPR) ^ xswz<DKP>(i);
        const unsigned voff = (i < nvalid && 8 * L < DK)
                                  ? (unsigned)(((size_t)(t0 + i) * a.H + h) * DK * 2 + 16 * L) : 0xFFFFFFF0u;
        mla::buf2lds16(c < NKC ? rk : rq, voff, smem + (c < NKC ? L::OFF_XK : L::OFF_XQ) + cc * 1024);
      } else {
        const int cc = c - 2 * NKC, i = GRK * cc + lane / GPR, c4 = 4 * (lane % GPR);
        const unsigned voff = (i < nvalid && c4 < DK)
                                  ? (unsigned)((((size_t)(t0 + i) * a.HV + hv) * DK + c4) * 4) : 0xFFFFFFF0u;
        mla::buf2lds16(rg, voff, smem + L::OFF_G + cc * 1024);
      }
    }
    // item r: row r % 64, channels 8 (r / 64) .. (consecutive lanes take consecutive
    // rows, so the transposed LDS writes below fall in distinct banks)
#pragma unroll
    for (int u = 0; u < VPER; ++u) {
      const int r = tid + NT * u, i = r % kC, c8 = 8 * (r / kC);
      vreg[u] = (r < NV && i < nvalid) ? *(const bf16x8*)(a.v + (((size_t)b * a.T + t0 + i) * a.HV + hv) * DV + c8)
                                       : bf16x8{};
    }
    if (tid < kC) sBeta[tid] = tid < nvalid ? a.beta[((size_t)b * a.T + t0 + tid) * a.HV + hv] : 0.0f;
    mla::wait_vmcnt<0>();
  }
  lds_barrier();

  // ---- phase 1: NT / DKP threads per key channel, each over RPT rows.  The
  // running Gam is kept for the thread's own rows, the 16-row block bounds
  // of those rows, the chunk end and (part 0) every block bound.
  constexpr int TPC = NT / DKP, RPT = kC / TPC;
  static_assert(NT % DKP == 0 && RPT % 8 == 0 && (RPT % 16 == 0 || 16 % RPT == 0), "row runs");
  const int ch = tid % DKP, part = tid / DKP;
  const int blk = (part * RPT) / 16;  // the 16-row block holding this thread's rows
  float own[RPT], ref0 = 0.0f, ref15 = 0.0f, gl = 0.0f, gs[4], ge[4];
  {
    float run = 0.0f;
#pragma unroll
    for (int i = 0; i < kC; ++i) {
      run += sG[i * DKP + ch];
      if (i / RPT == part) own[i % RPT] = run;
      if (i % 16 == 0) {
        gs[i / 16] = run;
        if (i / 16 == blk) ref0 = run;
      }
      if (i % 16 == 15) {
        ge[i / 16] = run;
        if (i / 16 == blk) ref15 = run;
      }
    }
    gl = run;
  }
  lds_barrier();  // R3 is free: Y and F may be written
  bf16x8 ktreg[RPT / 8];
  {
    const bool live = ch < DK;
    if (part == 0) Gimg[ch] = live ? exp_(gl) : 1.0f;
    // every read of this thread's k and q values goes out before the first
    // in-place write (the writes would otherwise order each row's reads)
    bf16 kraw[RPT], qraw[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int i = part * RPT + r;
      kraw[r] = *(const bf16*)(smem_raw + L::OFF_XK + xoff<DKP>(i, ch));
      qraw[r] = *(const bf16*)(smem_raw + L::OFF_XQ + xoff<DKP>(i, ch));
    }
#pragma unroll
    for (int i8 = 0; i8 < RPT / 8; ++i8) {
      bf16x8 at8;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = 8 * i8 + u, i = part * RPT + r;
        const float gm = own[r];
        bf16* pk = (bf16*)(smem_raw + L::OFF_XK + xoff<DKP>(i, ch));
        bf16* pq = (bf16*)(smem_raw + L::OFF_XQ + xoff<DKP>(i, ch));
        const float kk = (float)kraw[r], qq = (float)qraw[r];
        const float bi = sBeta[i];
        const float e = exp_(gm);
        ktreg[i8][u] = (bf16)(kk * e);
        at8[u] = (bf16)(bi * kk * exp_(gl - gm));
        const float eb = exp_(gm - ref0);
        *pk = (bf16)(kk * eb);
        *pq = (bf16)(qq * eb);
        sY[i * WP + ch] = (bf16)(bi * kk * exp_(ref15 - gm));
        Qimg[i * WP + ch] = (bf16)(qq * e);
      }
      *(bf16x8*)&Atimg[ch * TP + part * RPT + 8 * i8] = at8;
    }
    if (part == 0) {
      int p = 0;
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int J = 0; J <= I; ++J) sF[(p++) * DKP + ch] = exp_(gs[I] - ge[J]);
    }
  }
  lds_barrier();

  // ---- phase 2: A and Bm by 16-row block rows I (blocks J <= I).  With 8
  // waves, wave I forms A's row I and wave 4 + I Bm's; with 4, wave I both.
  const int bw = w & 3;
  const bool doA = NW == 4 || w < 4, doB = NW == 4 || w >= 4;
  f32x4 accA[4], accB[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) accA[J] = accB[J] = f32x4{};
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    if (J > bw) continue;
    const int pair = bw * (bw + 1) / 2 + J;
#pragma unroll
    for (int ks = 0; ks < DKP / 32; ++ks) {
      const int c0 = 32 * ks + 8 * kq;
      const bf16x8 y = lds8(smem, L::OFF_Y + ((16 * J + l16) * WP + c0) * 2);
      const f32x4 f0 = *(const f32x4*)&sF[pair * DKP + c0];
      const f32x4 f1 = *(const f32x4*)&sF[pair * DKP + c0 + 4];
      if (doA) {
        const bf16x8 xk = lds8(smem, L::OFF_XK + xoff<DKP>(16 * bw + l16, c0));
        bf16x8 xk2;
#pragma unroll
        for (int u = 0; u < 8; ++u) xk2[u] = (bf16)((float)xk[u] * (u < 4 ? f0[u] : f1[u - 4]));
        accA[J] = mla::mfma16(xk2, y, accA[J]);
      }
      if (doB) {
        const bf16x8 xq = lds8(smem, L::OFF_XQ + xoff<DKP>(16 * bw + l16, c0));
        bf16x8 xq2;
#pragma unroll
        for (int u = 0; u < 8; ++u) xq2[u] = (bf16)((float)xq[u] * (u < 4 ? f0[u] : f1[u - 4]));
        accB[J] = mla::mfma16(xq2, y, accB[J]);
      }
    }
  }
  // Bm image (rows i = 16 bw + 4 kq + e, column j = 16 J + l16), zero above the diagonal
  if (doB) {
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * bw + 4 * kq + e, j = 16 * J + l16;
        Bimg[i * TP + j] = (bf16)(j <= i ? accB[J][e] : 0.0f);
      }
  }
  lds_barrier();  // every wave is done with XK / XQ / Y / F
  if (doA) {
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * bw + 4 * kq + e, j = 16 * J + l16;
        sA[i * AP + j] = j < i ? accA[J][e] : 0.0f;
      }
  }
  lds_barrier();

  // ---- phase 3: Tm = (I + A)^{-1} by 16 x 16 blocks, fp32.  Waves 0-3
  // invert their diagonal block by forward substitution (lane c < 16:
  // column c); then, by distance d = I - J = 1, 2, 3, wave J forms
  //   T_IJ = -T_II sum_{M=J}^{I-1} A_IM T_MJ
  // (each lane 4 of the 256 elements, the sum staged in the wave's scratch).
  if (w < 4) {
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = (r == l16) ? 1.0f : 0.0f;
#pragma unroll
      for (int s2 = 0; s2 < r; ++s2) acc -= sA[(16 * w + r) * AP + 16 * w + s2] * x[s2];
      x[r] = acc;
    }
    if (lane < 16) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sTf[(16 * w + r) * AP + 16 * w + lane] = x[r];
    }
  }
  lds_barrier();
  float* sP = (float*)(smem_raw + L::OFF_P) + (w & 3) * 256;
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    if (w < 4 - d) {
      const int J = w, I = w + d;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int e = lane + 64 * m, i = e >> 4, j = e & 15;
        float acc = 0.0f;
        for (int M = J; M < I; ++M)
#pragma unroll
          for (int k2 = 0; k2 < 16; ++k2) acc += sA[(16 * I + i) * AP + 16 * M + k2] * sTf[(16 * M + k2) * AP + 16 * J + j];
        sP[e] = acc;
      }
      mla::wait_lgkmcnt0();
      asm volatile("" ::: "memory");
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int e = lane + 64 * m, i = e >> 4, j = e & 15;
        float acc = 0.0f;
#pragma unroll
        for (int k2 = 0; k2 < 16; ++k2) acc += sTf[(16 * I + i) * AP + 16 * I + k2] * sP[k2 * 16 + j];
        sTf[(16 * I + i) * AP + 16 * J + j] = -acc;
      }
    }
    lds_barrier();
  }
  // bf16 Tm for the MFMA products (zero above the diagonal blocks)
  for (int e = tid; e < kC * kC; e += NT) {
    const int i = e >> 6, j = e & 63;
    sT[i * TP + j] = (bf16)((j >> 4) > (i >> 4) ? 0.0f : sTf[i * AP + j]);
  }
  lds_barrier();  // A and the fp32 Tm are dead: K~^T and V^T may be written
#pragma unroll
  for (int i8 = 0; i8 < RPT / 8; ++i8) *(bf16x8*)&sKt[ch * TP + part * RPT + 8 * i8] = ktreg[i8];
#pragma unroll
  for (int u = 0; u < VPER; ++u) {
    const int r = tid + NT * u, i = r % kC, c8 = 8 * (r / kC);
    if (r < NV) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sVt[(c8 + e) * TP + i] = vreg[u][e];
    }
  }
  lds_barrier();

  // ---- phase 4: W^T = (k e^Gam)^T Tm^T (tiles: 16 channels x 16 rows) and
  // U = Tm V (tiles: 16 rows x 16 value channels)
  constexpr int NWT = (DKP / 16) * 4, NUT = 4 * (DV / 16);
  for (int tile = w; tile < NWT + NUT; tile += NW) {
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
// One bf16 store through a raw buffer descriptor: an offset at or past the
// descriptor's size writes nothing.  Issued from assembly so that every call
// is exactly one vector memory operation (the state kernel's wait counts rely
// on it).
__device__ __forceinline__ void buf_store_b16(const u32x4& rs, unsigned voff, bf16 v) {
  const unsigned d = (unsigned)__builtin_bit_cast(unsigned short, v);
  asm volatile("buffer_store_short %0, %1, %2, 0 offen" : : "v"(d), "v"(voff), "s"(rs) : "memory");
}

// Copies NB bytes (a multiple of 16) from global src into LDS dst: 1 KiB
// pieces, piece p issued by wave p % NW, the lanes of a last partial piece
// past NB masked off (so nothing past dst + NB is written).
template <int NB, int NW>
__device__ __forceinline__ void copy_image(const char* src, MLA_LDS char* dst, int w, int lane) {
  static_assert(NB % 16 == 0, "16-byte pieces");
  constexpr int PIECES = (NB + 1023) / 1024;
  const u32x4 rs = mla::make_rsrc(src, (unsigned)NB);
#pragma unroll
  for (int p = 0; p < PIECES; ++p) {
    if (p % NW != w) continue;
    if (p * 1024 + 16 * lane < NB) mla::buf2lds16(rs, (unsigned)(p * 1024 + 16 * lane), dst + p * 1024);
  }
}

template <int DK, int DV, int VB>
struct StateLds {
  using D = KdaDims<DK, DV>;
  // double-buffered per chunk: W, q e^Gam, A_hat^T, Bm, the chunk decay
  static constexpr int S_W = 0;
  static constexpr int S_Q = S_W + D::W_BYTES;
  static constexpr int S_AT = S_Q + D::W_BYTES;
  static constexpr int S_B = S_AT + D::AT_BYTES;
  static constexpr int S_G = S_B + D::B_BYTES;
  static constexpr int STAGE = round_up(S_G + D::G_BYTES, 16);
  // single-buffered: this block's U^T rows (refilled once R has used them)
  static constexpr int UT_SLICE = VB * D::TP * 2;
  static constexpr int OFF_UT = 2 * STAGE;
  static constexpr int OFF_ST = OFF_UT + UT_SLICE;              // S^T bf16 [VB][WP]
  static constexpr int OFF_RT = OFF_ST + VB * D::WP * 2;        // R^T bf16 [VB][TP]
  static constexpr int BYTES = OFF_RT + VB * D::TP * 2;
  static_assert(BYTES <= 163840, "LDS");
};

// One workgroup (NW = 4 or 8 waves) per (batch, value head, VB value
// columns).  Wave w owns rows 16 (w % 4) .. of R and O and channel tiles
// w % 4, w % 4 + 4, ... of S, over the value tiles of its share: all of them
// with 4 waves, half (w / 4 picks which) with 8.  Eight waves put two on each
// SIMD, so one wave's LDS reads and MFMA chains run while the other waits.
template <int DK, int DV, int VB, int NW>
__global__ void __launch_bounds__(64 * NW) kda_state(KdaArgs a) {
  using D = KdaDims<DK, DV>;
  using L = StateLds<DK, DV, VB>;
  constexpr int DKP = D::DKP, WP = D::WP, TP = D::TP;
  constexpr int NVB = DV / VB, NVT = VB / 16, NCT = DKP / 16, CPW = (NCT + 3) / 4;
  constexpr int NVW = NVT / (NW / 4);  // value tiles per wave
  static_assert(DV % VB == 0 && VB % 16 == 0, "value blocks");
  static_assert((NW == 4 || NW == 8) && NVT % (NW / 4) == 0, "waves split the value tiles evenly");
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
  const int wr = w & 3, V0 = (w >> 2) * NVW;  // row block / channel tile base; first value tile
  const int l16 = lane & 15, kq = lane >> 4;
  const int v0 = vb * VB;

  auto slot_of = [&](int ci) { return a.ws + ((size_t)bh * a.NC + ci) * D::SLOT; };
  auto issue_main = [&](int ci, int st) {
    const char* slot = slot_of(ci);
    MLA_LDS char* dst = smem + st * L::STAGE;
    copy_image<D::W_BYTES, NW>(slot + D::OFF_W, dst + L::S_W, w, lane);
    copy_image<D::W_BYTES, NW>(slot + D::OFF_Q, dst + L::S_Q, w, lane);
    copy_image<D::AT_BYTES, NW>(slot + D::OFF_AT, dst + L::S_AT, w, lane);
    copy_image<D::B_BYTES, NW>(slot + D::OFF_B, dst + L::S_B, w, lane);
    copy_image<D::G_BYTES, NW>(slot + D::OFF_G, dst + L::S_G, w, lane);
  };
  auto issue_ut = [&](int ci) {
    copy_image<L::UT_SLICE, NW>(slot_of(ci) + D::OFF_UT + v0 * TP * 2, smem + L::OFF_UT, w, lane);
  };
  issue_main(0, 0);
  issue_ut(0);

  // the state: fragment (m, vv) holds channels 16 (wr + 4 m) + 4 kq + e of
  // value column 16 (V0 + vv) + l16
  f32x4 S[CPW][NVW];
#pragma unroll
  for (int m = 0; m < CPW; ++m) {
    const int C = wr + 4 * m;
#pragma unroll
    for (int vv = 0; vv < NVW; ++vv) {
      const int V = V0 + vv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 16 * C + 4 * kq + e;
        S[m][vv][e] = (a.s0 && C < NCT && c < DK)
                         ? a.s0[(((size_t)b * a.HV + hv) * DK + c) * DV + v0 + 16 * V + l16]
                         : 0.0f;
      }
      if (C < NCT) {
        bf16x4 s4;
#pragma unroll
        for (int e = 0; e < 4; ++e) s4[e] = (bf16)S[m][vv][e];
        *(bf16x4*)&sSt[(16 * V + l16) * WP + 16 * C + 4 * kq] = s4;
      }
    }
  }

  // O is written with NVW * 4 buffer stores per wave and chunk, always issued
  // (rows past T fall outside the descriptor and are dropped), so the wait
  // for chunk ci's copies can leave the previous chunk's stores in flight:
  // vector memory operations complete in issue order, and those stores are
  // the youngest.
  constexpr int OST = NVW * 4;
  static_assert(OST < 64, "vmcnt range");
  for (int ci = 0; ci < a.NC; ++ci) {
    if (ci == 0) mla::wait_vmcnt<0>();
    else mla::wait_vmcnt<OST>();
    mla::wait_lgkmcnt0();
    mla::wg_barrier();  // chunk ci staged, S^T of the previous chunk written, R^T free
    if (ci + 1 < a.NC) issue_main(ci + 1, (ci + 1) & 1);
    const int so = (ci & 1) * L::STAGE;

    // R = U - W S and P = (q e^Gam) S: rows 16 wr + 4 kq + e, value column
    // 16 (V0 + vv) + l16
    f32x4 accR[NVW], accP[NVW];
#pragma unroll
    for (int vv = 0; vv < NVW; ++vv) accR[vv] = accP[vv] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < DKP / 32; ++ks) {
      const int c0 = 32 * ks + 8 * kq;
      const bf16x8 aw = lds8(smem, so + L::S_W + ((16 * wr + l16) * WP + c0) * 2);
      const bf16x8 aq = lds8(smem, so + L::S_Q + ((16 * wr + l16) * WP + c0) * 2);
#pragma unroll
      for (int vv = 0; vv < NVW; ++vv) {
        const bf16x8 bs = lds8(smem, L::OFF_ST + ((16 * (V0 + vv) + l16) * WP + c0) * 2);
        accR[vv] = mla::mfma16(aw, bs, accR[vv]);
        accP[vv] = mla::mfma16(aq, bs, accP[vv]);
      }
    }
#pragma unroll
    for (int vv = 0; vv < NVW; ++vv) {
      const int V = V0 + vv;
      const bf16x4 u4 = *(const MLA_LDS bf16x4*)(smem + L::OFF_UT + ((16 * V + l16) * TP + 16 * wr + 4 * kq) * 2);
      bf16x4 r4;
#pragma unroll
      for (int e = 0; e < 4; ++e) r4[e] = (bf16)((float)u4[e] - accR[vv][e]);
      *(bf16x4*)&sRt[(16 * V + l16) * TP + 16 * wr + 4 * kq] = r4;
    }
    mla::wait_lgkmcnt0();
    mla::wg_barrier();  // R^T complete; every wave is done reading S^T and U^T
    if (ci + 1 < a.NC) issue_ut(ci + 1);

    // O = P + Bm R
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int j0 = 32 * ks + 8 * kq;
      const bf16x8 ab = lds8(smem, so + L::S_B + ((16 * wr + l16) * TP + j0) * 2);
#pragma unroll
      for (int vv = 0; vv < NVW; ++vv)
        accP[vv] = mla::mfma16(ab, lds8(smem, L::OFF_RT + ((16 * (V0 + vv) + l16) * TP + j0) * 2), accP[vv]);
    }
    {
      // rows t0 .. min(t0 + 64, T) - 1 of this head; a row at or past T lies
      // past the descriptor's last byte
      const int t0 = ci * kC;
      const int rows = min(kC, a.T - t0);
      const u32x4 rs = mla::make_rsrc(a.o + ((size_t)b * a.T + t0) * a.HV * DV, (unsigned)(rows * a.HV * DV * 2));
#pragma unroll
      for (int vv = 0; vv < NVW; ++vv)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * wr + 4 * kq + e;
          buf_store_b16(rs, (unsigned)(((r * a.HV + hv) * DV + v0 + 16 * (V0 + vv) + l16) * 2), (bf16)accP[vv][e]);
        }
    }

    // S = e^{Gam_63} S + A_hat^T R
#pragma unroll
    for (int m = 0; m < CPW; ++m) {
      const int C = wr + 4 * m;
      if (C >= NCT) continue;
      const f32x4 gc = *(const MLA_LDS f32x4*)(smem + so + L::S_G + (16 * C + 4 * kq) * 4);
#pragma unroll
      for (int vv = 0; vv < NVW; ++vv)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[m][vv][e] *= gc[e];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int j0 = 32 * ks + 8 * kq;
        const bf16x8 aa = lds8(smem, so + L::S_AT + ((16 * C + l16) * TP + j0) * 2);
#pragma unroll
        for (int vv = 0; vv < NVW; ++vv)
          S[m][vv] = mla::mfma16(aa, lds8(smem, L::OFF_RT + ((16 * (V0 + vv) + l16) * TP + j0) * 2), S[m][vv]);
      }
#pragma unroll
      for (int vv = 0; vv < NVW; ++vv) {
        bf16x4 s4;
#pragma unroll
        for (int e = 0; e < 4; ++e) s4[e] = (bf16)S[m][vv][e];
        *(bf16x4*)&sSt[(16 * (V0 + vv) + l16) * WP + 16 * C + 4 * kq] = s4;
      }
    }
  }

  if (a.s_out) {
#pragma unroll
    for (int m = 0; m < CPW; ++m) {
      const int C = wr + 4 * m;
      if (C >= NCT) continue;
#pragma unroll
      for (int vv = 0; vv < NVW; ++vv)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = 16 * C + 4 * kq + e;
          if (c < DK) a.s_out[(((size_t)b * a.HV + hv) * DK + c) * DV + v0 + 16 * (V0 + vv) + l16] = S[m][vv][e];
        }
    }
  }
}

}  // namespace kda
