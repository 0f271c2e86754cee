// bf16 backward of the absorbed Gated MLA prefill core on gfx950.  The pages
// train the layer with a cross-entropy loss; the gradients are the chain rule
// through the forward of page "Gated MLA（矩阵吸收版）", section
// 完整计算流（四步） (absorb, latent score, causal softmax, latent sum, W_UV,
// sigmoid gate).  With a = q W_UK (absorbed query), P the causal softmax of
// S = scale a c^T, ol = P c and o = ol W_UV^T, given dout:
//
//   dg = dout * out * (1 - sigmoid(g))          do = dout * sigmoid(g)
//   dol = do W_UV                               D_t = sum_v dout out  (= dol . ol)
//   dS = P (dol c^T - D)                        da = scale dS c
//   dc = scale dS^T a + P^T dol                 dq = da W_UK^T
//   dW_UK = sum_t q_t^T da_t                    dW_UV = sum_t do_t^T ol_t = sum_s dV_s^T c_s
// with dV_s = sum_t P_ts do_t (the value gradient of the decompressed form).
//
// Kernels (in call order):
//   mla_bwd_prep     dg, do and the per-row pair {lse log2 e, D}
//   GEMMs            q_abs2 = scale log2e q W_UK and dol = do W_UV, head-major
//   mla_bwd_query    per (32 queries, head): da over the key tiles
//   mla_bwd_key      per (64 keys, head group): partial dc and, per head, dV
//                    over the query blocks at or after the keys
//   mla_bwd_dc_sum   dc = sum of the head-group partials
//   GEMMs            dq = da W_UK^T (NT), dW_UK = q^T da and dW_UV = dV^T c (TN)
//
// Head-major rows: q_abs2, dol and da are [H, B*T, R], do and dV [H, B*T, DV],
// so the 32 rows of one (head, block) are one contiguous 32-row tile, copied
// like a latent tile.  The scores of the forward are recomputed from q_abs2 and c with the
// forward's log-sum-exp, P = exp2(S2 - lse log2 e).
#pragma once

#include "attn_core.h"

namespace mla {

struct BwdArgs {
  const bf16* c;      // [B, T, R]
  const bf16* qabs;   // [H, B*T, R]  scale * log2(e) * q W_UK
  const bf16* dolat;  // [H, B*T, R]  do W_UV
  const float* ld;    // [H, B*T, 2]  {lse * log2(e), D}
  const bf16* dov;    // [H, B*T, DV] do = dout * sigmoid(g)
  bf16* da;           // [H, B*T, R]
  bf16* dv;           // [H, B*T, DV] dV
  float* dc_part;     // [nhg, B*T, R]
  int B, T, H;
  float scale;
  int ntb;            // ceil(T / 32)
  int nhg, hpg;       // head groups of mla_bwd_key and heads per group
};

constexpr int kBwdWaves = 8;
constexpr int kXPitch = 33;  // fp32 exchange rows (floats)
constexpr int kPPitch = 40;  // bf16 P / dS rows (elements): 80-byte rows keep b128 reads aligned

// Exchange buffers after the tile stages: S and dP (fp32 [32][33] each), P and
// dS (bf16 [32][40] each).
constexpr int kBwdXBytes = 2 * 32 * kXPitch * 4 + 2 * 32 * kPPitch * 2;

// Transposed operand of a stored 32-row tile (rows = the reduction index):
// lane l gets rows 8 (l/16) + 0..7 of column 16 jt + l % 16.
template <int R>
__device__ __forceinline__ bf16x8 tile_column_operand(const MLA_LDS char* tile, int jt, int l16, int kq) {
  const int e = l16 >> 2, q = l16 & 3;
  const int chunk = 2 * jt + (q >> 1), half = (q & 1) * 8;
  const MLA_LDS char* p0 = tile + tile_off<R>(8 * kq + e, chunk) + half;
  const MLA_LDS char* p1 = tile + tile_off<R>(8 * kq + 4 + e, chunk) + half;
  return cat4(lds_read_tr16(p0), lds_read_tr16(p1));
}

// ----------------------------------------------------------------- prep
struct BwdPrepArgs {
  const bf16* gate;   // [B*T, H*DV]
  const bf16* out;    // [B*T, H*DV]  forward output
  const bf16* dout;   // [B*T, H*DV]
  const float* lse;   // [B, H, T]    forward log-sum-exp (natural log)
  bf16* dgate;        // [B*T, H*DV], rows ldg apart
  bf16* dov;          // [H, B*T, DV] do = dout * sigmoid(g)
  float* ld;          // [H, B*T, 2]
  int B, T, H, DV, ldg;
};

// One workgroup per token row; wave w takes heads w, w+4, ...; lanes walk the
// DV values of a head.  The heads go in batches of HB whose loads are all
// issued before the batch's first store: the stores may alias the loads as
// far as the compiler knows, so a loop storing head by head would wait one
// memory round trip per head.
template <int DV>
__global__ void __launch_bounds__(256) mla_bwd_prep(BwdPrepArgs a) {
  constexpr int NV = (DV + 63) / 64;  // values per lane and head
  constexpr int HB = 6;               // heads per batch of loads
  const int bt = blockIdx.x, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = bt / a.T, t = bt % a.T;
  const size_t row = (size_t)bt * a.H * DV;
  for (int hb = w; hb < a.H; hb += 4 * HB) {
    float g[HB][NV], o[HB][NV], d[HB][NV], lse[HB];
#pragma unroll
    for (int u = 0; u < HB; ++u) {
      // clamped addresses: every load is issued, none behind a branch
      const int hc = min(hb + 4 * u, a.H - 1);
      lse[u] = a.lse[((size_t)b * a.H + hc) * a.T + t];
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const size_t i = row + (size_t)hc * DV + min(lane + 64 * j, DV - 1);
        g[u][j] = (float)a.gate[i];
        o[u][j] = (float)a.out[i];
        d[u][j] = (float)a.dout[i];
      }
    }
#pragma unroll
    for (int u = 0; u < HB; ++u) {
      const int h = hb + 4 * u;
      if (h >= a.H) break;  // wave-uniform
      float dsum = 0.0f;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int v = lane + 64 * j;
        if (v < DV) {
          const float s = sigmoidf_(g[u][j]);
          a.dgate[(size_t)bt * a.ldg + (size_t)h * DV + v] = (bf16)(d[u][j] * o[u][j] * (1.0f - s));
          a.dov[((size_t)h * a.B * a.T + bt) * DV + v] = (bf16)(d[u][j] * s);
          dsum += d[u][j] * o[u][j];
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) dsum += __shfl_xor(dsum, off, 64);
      if (lane == 0) {
        float* dst = a.ld + ((size_t)h * a.B * a.T + bt) * 2;
        dst[0] = lse[u] * kLog2e;
        dst[1] = dsum;
      }
    }
  }
}

// ----------------------------------------------------------------- query side
// Workgroup (batch b, 32 queries t0.., head h), 8 waves, heaviest blocks
// first.  A step covers 64 keys (two 32-row latent tiles per LDS stage, two
// stages, one step of lookahead).  Wave w owns the 16x16 tile (queries
// 16 (w%2) .., keys 16 (w/2) ..) of both S2 = q_abs2 c^T and dP = dol c^T:
// the key rows of c are the shared B operand, the wave's q_abs2 and dol rows
// are its A operands (held in VGPRs), so P and dS are formed in registers and
// written once as query-major bf16 rows.  Wave w then accumulates da^T for
// latent tiles w, w+8, ...: da^T += c^T dS^T over the 64 keys, c^T from
// transposing reads of the tiles.
constexpr int kBwdQKeys = 64;
constexpr int kDSPitch = kBwdQKeys + 8;  // bf16 dS rows (elements), 144 bytes

template <int R>
__global__ void __launch_bounds__(64 * kBwdWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
mla_bwd_query(BwdArgs a) {
  using LT = LatentTile<R>;
  constexpr int NKK = R / 32, NJT = R / 16;
  constexpr int JPW = (NJT + kBwdWaves - 1) / kBwdWaves;
  constexpr int SUB = kBwdQKeys / LT::KT;  // latent tiles per step
  constexpr int STAGE = SUB * LT::BYTES;
  static_assert(LT::COPIES % kBwdWaves == 0 || LT::COPIES < kBwdWaves, "copy split");
  static_assert(SUB == 2, "two 32-row tiles per step");
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * STAGE + 32 * kDSPitch * 2];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;
  bf16* dSb = (bf16*)(smem_raw + 2 * STAGE);

  const int x = blockIdx.x;
  const int h = x % a.H, rest = x / a.H;
  const int b = rest % a.B, tb = a.ntb - 1 - rest / a.B;
  const int T = a.T, t0 = tb * 32;
  const int nsteps = (min(t0 + 32, T) + kBwdQKeys - 1) / kBwdQKeys;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, kq = lane >> 4;
  const int qt = w & 1, kt = w >> 1;  // query tile, 16-key tile of the step
  const size_t hrow = (size_t)h * a.B * T + (size_t)b * T;  // head-major row of (b, t = 0)

  // A operands: query rows 16 qt + l16 of q_abs2 and dol
  bf16x8 aq[NKK], ad[NKK];
  {
    const size_t row = (hrow + min(t0 + 16 * qt + l16, T - 1)) * R + 8 * kq;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      aq[kk] = *(const bf16x8*)(a.qabs + row + 32 * kk);
      ad[kk] = *(const bf16x8*)(a.dolat + row + 32 * kk);
    }
  }
  // {lse log2 e, D} of this lane's fragment rows: queries 16 qt + 4 kq + i
  float L2[4], Dq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float* p = a.ld + (hrow + min(t0 + 16 * qt + 4 * kq + i, T - 1)) * 2;
    L2[i] = p[0];
    Dq[i] = p[1];
  }

  f32x4 acc[JPW][2];
#pragma unroll
  for (int j = 0; j < JPW; ++j) acc[j][0] = acc[j][1] = f32x4{};

  TileCopier<R, kBwdWaves> copier;
  copier.init(w, lane);
  const bf16* cb = a.c + (size_t)b * T * R;
  auto issue_step = [&](int it, MLA_LDS char* dst) {
#pragma unroll
    for (int u = 0; u < SUB; ++u) copier.issue(cb, it * kBwdQKeys + u * LT::KT, T, dst + u * LT::BYTES);
  };
  issue_step(0, smem);

  for (int it = 0; it < nsteps; ++it) {
    wait_vmcnt<0>();
    wg_barrier();  // step it staged; the previous step's update is done everywhere
    if (it + 1 < nsteps) issue_step(it + 1, smem + ((it + 1) & 1) * STAGE);
    const MLA_LDS char* st = smem + (it & 1) * STAGE;
    const MLA_LDS char* ktile = st + (kt >> 1) * LT::BYTES;  // the 32-row tile holding key tile kt

    // S2 and dP tile (qt, kt): rows query 16 qt + 4 kq + i, column key 16 kt + l16
    f32x4 sacc = f32x4{}, dacc = f32x4{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const bf16x8 bk = lds_read_b128(ktile + tile_off<R>(16 * (kt & 1) + l16, 4 * kk + kq));
      sacc = mfma16(aq[kk], bk, sacc);
      dacc = mfma16(ad[kk], bk, dacc);
    }
    {
      const int kc = 16 * kt + l16, kpos = it * kBwdQKeys + kc;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qr = 16 * qt + 4 * kq + i, qpos = t0 + qr;
        const float p = (kpos <= qpos) ? fast_exp2(sacc[i] - L2[i]) : 0.0f;
        dSb[qr * kDSPitch + kc] = (bf16)(p * (dacc[i] - Dq[i]));
      }
    }
    wait_lgkmcnt0();
    wg_barrier();

    // da^T += c^T [16 latent x 32 keys] x dS^T [32 keys x 16 queries], two key halves
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      bf16x8 bS[2];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) bS[c2] = *(const bf16x8*)&dSb[(16 * c2 + l16) * kDSPitch + 32 * u + 8 * kq];
#pragma unroll
      for (int j = 0; j < JPW; ++j) {
        const int jt = w + kBwdWaves * j;
        if (jt < NJT) {
          const bf16x8 ac = tile_column_operand<R>(st + u * LT::BYTES, jt, l16, kq);
          acc[j][0] = mfma16(ac, bS[0], acc[j][0]);
          acc[j][1] = mfma16(ac, bS[1], acc[j][1]);
        }
      }
    }
  }

  // epilogue: fragment (j, c2) holds latent dims 16 jt + 4 kq + e of query 16 c2 + l16
#pragma unroll
  for (int j = 0; j < JPW; ++j) {
    const int jt = w + kBwdWaves * j;
    if (jt >= NJT) continue;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int tq = t0 + 16 * c2 + l16;
      if (tq >= T) continue;
      bf16x4 vd;
#pragma unroll
      for (int e = 0; e < 4; ++e) vd[e] = (bf16)(acc[j][c2][e] * a.scale);
      *(bf16x4*)(a.da + (hrow + tq) * R + 16 * jt + 4 * kq) = vd;
    }
  }
}

// ----------------------------------------------------------------- key side
// Workgroup (batch b, 64 keys k0.., head group hg), 8 waves, blocks with the
// most query blocks first.  Steps run over (head h of the group, 32-query
// block qb from the one holding key k0 on); a step stages the q_abs2 and dol
// tiles of (h, qb) and their {lse log2 e, D} pairs in LDS (two stages, one
// step of lookahead).  Wave w owns the 16x16 tile (keys 16 (w/2) .., queries
// 16 (w%2) ..) of both S2^T and dP^T: the key rows of c are its MFMA A
// operand for both products (held in VGPRs), so P and dS ln 2 are formed in
// registers and written once as key-major bf16 rows.  Wave w then
// accumulates dc^T for latent tiles w, w+8, ... over all 64 keys:
//   dc^T += q_abs2^T (dS ln 2)^T + dol^T P^T
// (q_abs2 carries scale log2 e, so dS ln 2 gives the scale dS a term), and
// dV^T for value tile w: dV^T += do^T P^T, stored per head when the head's
// last query block is done (do is staged with the step's tiles).
constexpr int kBwdKeys = 64;

template <int DV, int R>
struct BwdKeyConfig {
  static constexpr int LDB = 256;                                    // {L2, D} x 32 queries
  static constexpr int DOB = LatentTile<DV>::BYTES;                  // do tile, 32 x DV
  static constexpr int STAGE = 2 * LatentTile<R>::BYTES + DOB + LDB;
  static constexpr int PBYTES = kBwdKeys * kPPitch * 2;             // one bf16 [64][40] array
  static constexpr int LDS = 2 * STAGE + 2 * PBYTES;
};

template <int DV, int R>
__global__ void __launch_bounds__(64 * kBwdWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
mla_bwd_key(BwdArgs a) {
  using LT = LatentTile<R>;
  using LV = LatentTile<DV>;
  using CFG = BwdKeyConfig<DV, R>;
  constexpr int NVT = DV / 16;  // value tiles: wave w < NVT owns tile w
  constexpr int NKK = R / 32, NJT = R / 16;
  constexpr int JPW = (NJT + kBwdWaves - 1) / kBwdWaves;
  constexpr int KTS = kBwdKeys / 16;  // 16-key tiles
  static_assert(LT::COPIES % kBwdWaves == 0 || LT::COPIES < kBwdWaves, "copy split");
  static_assert(KTS * 2 == kBwdWaves, "one (key tile, query tile) pair per wave");
  static_assert(NVT <= kBwdWaves, "one value tile per wave at most");
  static_assert(LV::COPIES % kBwdWaves == 0 || LV::COPIES < kBwdWaves, "copy split");
  __shared__ __attribute__((aligned(1024))) char smem_raw[CFG::LDS];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;
  bf16* Pb = (bf16*)(smem_raw + 2 * CFG::STAGE);
  bf16* dSb = Pb + kBwdKeys * kPPitch;

  const int x = blockIdx.x;
  const int hg = x % a.nhg, rest = x / a.nhg;
  const int b = rest % a.B, kb = rest / a.B;
  const int T = a.T, k0 = kb * kBwdKeys;
  const int h0 = hg * a.hpg, nh = min(a.hpg, a.H - h0);
  const int qb0 = k0 / 32;
  const int nq = a.ntb - qb0;
  const int nsteps = nh * nq;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, kq = lane >> 4;
  const int kt = w >> 1, qt = w & 1;
  const size_t BT = (size_t)a.B * T;

  // A operand: key rows 16 kt + l16 of c
  bf16x8 aop[NKK];
  {
    const int tk = min(k0 + 16 * kt + l16, T - 1);
    const bf16* src = a.c + ((size_t)b * T + tk) * R + 8 * kq;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) aop[kk] = *(const bf16x8*)(src + 32 * kk);
  }

  f32x4 acc[JPW][KTS], accv[KTS];
#pragma unroll
  for (int j = 0; j < JPW; ++j)
#pragma unroll
    for (int t = 0; t < KTS; ++t) acc[j][t] = f32x4{};
#pragma unroll
  for (int t = 0; t < KTS; ++t) accv[t] = f32x4{};

  TileCopier<R, kBwdWaves> copier;
  copier.init(w, lane);
  TileCopier<DV, kBwdWaves> vcopier;
  vcopier.init(w, lane);
  auto stage = [&](int st) { return smem + st * CFG::STAGE; };
  auto issue_step = [&](int s, MLA_LDS char* dst) {
    const int h = h0 + s / nq, qb = qb0 + s % nq;
    const size_t r0 = (size_t)h * BT + (size_t)b * T;  // row t = 0 of (h, b)
    copier.issue(a.qabs + r0 * R, qb * 32, T, dst);
    copier.issue(a.dolat + r0 * R, qb * 32, T, dst + LT::BYTES);
    vcopier.issue(a.dov + r0 * DV, qb * 32, T, dst + 2 * LT::BYTES);
    if (w == 0 && lane < 16) {
      const int rows = min(32, T - qb * 32);
      const u32x4 rs = make_rsrc(a.ld + (r0 + qb * 32) * 2, (unsigned)(rows * 8));
      buf2lds16(rs, (unsigned)(lane * 16), dst + 2 * LT::BYTES + CFG::DOB);
    }
  };
  if (nsteps > 0) issue_step(0, stage(0));

  for (int s = 0; s < nsteps; ++s) {
    wait_vmcnt<0>();
    wg_barrier();  // step s staged; step s-1 done everywhere (its stage and the P / dS rows are free)
    if (s + 1 < nsteps) issue_step(s + 1, stage((s + 1) & 1));
    const MLA_LDS char* tq_tile = stage(s & 1);
    const MLA_LDS char* td_tile = tq_tile + LT::BYTES;
    const MLA_LDS char* tv_tile = td_tile + LT::BYTES;
    const float* ldst = (const float*)(smem_raw + (s & 1) * CFG::STAGE + 2 * LT::BYTES + CFG::DOB);
    const int qb = qb0 + s % nq;

    // S2^T and dP^T tile (kt, qt): rows key 16 kt + 4 kq + i, column query 16 qt + l16
    f32x4 sacc = f32x4{}, dacc = f32x4{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int off = tile_off<R>(16 * qt + l16, 4 * kk + kq);
      sacc = mfma16(aop[kk], lds_read_b128(tq_tile + off), sacc);
      dacc = mfma16(aop[kk], lds_read_b128(td_tile + off), dacc);
    }
    {
      const int q = 16 * qt + l16, qpos = qb * 32 + q;
      const float L2 = ldst[2 * q], Dq = ldst[2 * q + 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kr = 16 * kt + 4 * kq + i, kpos = k0 + kr;
        // a query past T has no {lse, D} pair of its own: the staged bytes
        // there may be anything, so both products are selected, not scaled, to zero
        const bool live = kpos <= qpos && qpos < T;
        const float p = live ? fast_exp2(sacc[i] - L2) : 0.0f;
        Pb[kr * kPPitch + q] = (bf16)p;
        dSb[kr * kPPitch + q] = live ? (bf16)(p * (dacc[i] - Dq) * 0.69314718055994531f) : (bf16)0.0f;
      }
    }
    wait_lgkmcnt0();
    wg_barrier();

    bf16x8 bS[KTS], bP[KTS];
#pragma unroll
    for (int t = 0; t < KTS; ++t) {
      bS[t] = *(const bf16x8*)&dSb[(16 * t + l16) * kPPitch + 8 * kq];
      bP[t] = *(const bf16x8*)&Pb[(16 * t + l16) * kPPitch + 8 * kq];
    }
#pragma unroll
    for (int j = 0; j < JPW; ++j) {
      const int jt = w + kBwdWaves * j;
      if (jt < NJT) {
        const bf16x8 aq = tile_column_operand<R>(tq_tile, jt, l16, kq);
        const bf16x8 ad = tile_column_operand<R>(td_tile, jt, l16, kq);
#pragma unroll
        for (int t = 0; t < KTS; ++t) {
          acc[j][t] = mfma16(aq, bS[t], acc[j][t]);
          acc[j][t] = mfma16(ad, bP[t], acc[j][t]);
        }
      }
    }
    if (w < NVT) {
      // dV^T [16 values x 64 keys] += do^T [16 values x 32 queries] P^T
      const bf16x8 av = tile_column_operand<DV>(tv_tile, w, l16, kq);
#pragma unroll
      for (int t = 0; t < KTS; ++t) accv[t] = mfma16(av, bP[t], accv[t]);
      if (s % nq == nq - 1) {
        // the head's last query block: store its dV rows (values 16 w + 4 kq + e of key 16 t + l16)
        const int h = h0 + s / nq;
        const size_t r0 = (size_t)h * BT + (size_t)b * T;
#pragma unroll
        for (int t = 0; t < KTS; ++t) {
          const int tk = k0 + 16 * t + l16;
          if (tk < T) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (bf16)accv[t][e];
            *(bf16x4*)(a.dv + (r0 + tk) * DV + 16 * w + 4 * kq) = v;
          }
          accv[t] = f32x4{};
        }
      }
    }
  }

  // epilogue: fragment (j, t) holds latent dims 16 jt + 4 kq + e of key 16 t + l16
#pragma unroll
  for (int j = 0; j < JPW; ++j) {
    const int jt = w + kBwdWaves * j;
    if (jt >= NJT) continue;
#pragma unroll
    for (int t = 0; t < KTS; ++t) {
      const int tk = k0 + 16 * t + l16;
      if (tk >= T) continue;
      *(f32x4*)(a.dc_part + ((size_t)hg * BT + (size_t)b * T + tk) * R + 16 * jt + 4 * kq) = acc[j][t];
    }
  }
}

// dc[row, :] = sum over head groups of the partials (bf16 out); one thread
// per 4 latent values.
__global__ void __launch_bounds__(256) mla_bwd_dc_sum(const float* __restrict__ part, bf16* __restrict__ dc,
                                                      long long rows, int R, int nhg) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;  // index of 4 values
  const long long n4 = rows * R / 4;
  if (i >= n4) return;
  f32x4 s = f32x4{};
  for (int g = 0; g < nhg; ++g) s += *(const f32x4*)(part + ((long long)g * rows * R) + 4 * i);
  bf16x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (bf16)s[e];
  *(bf16x4*)(dc + 4 * i) = v;
}

}  // namespace mla
