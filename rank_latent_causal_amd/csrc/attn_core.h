// Per-wave latent-attention core shared by the prefill and decode kernels.
//
// A wave owns 16 query rows (the N index of every MFMA, lane l serves row
// l % 16) and the full r-wide latent accumulator O^T [r x 16] in VGPRs.  One
// 32-key latent tile held in LDS (row-major, chunk-swizzled) is consumed as
//   S^T = c_tile . q_abs^T              (A = c rows via ds_read_b128)
//   P   = exp2(S - m), online softmax   (per-lane statistics)
//   O^T += c_tile^T . P^T               (A = c columns via ds_read_b64_tr_b16)
// Because the score uses the same latent rows as the values (K = V = c),
// a single LDS copy feeds both products.
//
// k-slot bookkeeping: lane (l16 = l % 16, kq = l / 16) of a C fragment holds
// rows 4 kq + e.  Two 16-row C fragments (rows 0-15 and 16-31) therefore give
// the lane the 8 values a B operand needs in k slots {4kq+e} and {16+4kq+e};
// the A operands are read with that same key order, so C fragments are fed
// back as B operands without any lane shuffle.
#pragma once

#include "common.h"

namespace mla {

template <int R>
struct LatentTile {
  static constexpr int KT = 32;             // keys per tile
  static constexpr int BYTES = KT * R * 2;  // bf16 row-major tile
  static constexpr int NKK = R / 32;        // score k-steps (32 latent dims)
  static constexpr int NJT = R / 16;        // value tiles (16 latent dims)
  static constexpr int COPIES = KT * (R / 8) / 64;  // 1 KiB wave copies per tile
};

template <int R>
constexpr int copies_per_wave(int nwaves) {
  return (LatentTile<R>::COPIES + nwaves - 1) / nwaves;
}

// Copies latent rows [row0, row0 + 32) into a swizzled LDS tile with raw
// buffer loads.  Copy qi (1 KiB of LDS, rows qi*RPI .. of the tile) is issued
// by wave qi % NW, so each wave issues either copies_per_wave(NW) copies or
// none.  One scalar descriptor covers the tile's valid rows, so rows at or
// past row_end read as zeros (their scores are masked).  The swizzle is
// XOR-linear in the row bits and a copy's first row is a multiple of its row
// count, so a lane's byte offset is a fixed per-lane base XOR a wave-uniform
// constant (swizzle term and row offset occupy disjoint bits): one VALU op
// per copy.
template <int R, int NW, int SW = 0>
struct TileCopier {
  static constexpr int COPIES = LatentTile<R>::COPIES;
  static constexpr int CPW = copies_per_wave<R>(NW);
  static constexpr int CPR = R / 8;       // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;    // rows per copy
  static constexpr int KT = LatentTile<R>::KT;
  static_assert(64 % CPR == 0, "a copy covers whole rows");
  int w;

  __device__ __forceinline__ void init(int wave, int /*lane*/) { w = wave; }

  // This lane's byte offset inside a copy.  The lane id is re-read with
  // v_mbcnt at every tile (from asm, so the result is not hoisted): a base
  // kept live across the whole key loop costs a VGPR in kernels that are at
  // the register limit, and a spilled base reloads behind a vmcnt(0) that
  // drains the tile prefetches.
  __device__ __forceinline__ unsigned lane_base() const {
    unsigned ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    const unsigned sl = ln / CPR;
    return (sl * R + (((ln % CPR) ^ (unsigned)tile_swizzle<R, SW>((int)sl)) * 8)) * 2;
  }

  // A tile's descriptor and this wave's copy offsets, formed once; the
  // copies themselves can then be issued in several groups (issue_range), so
  // a wave does not stall on a full vector-memory queue by sending all of
  // them at once.
  struct Pending {
    u32x4 rs;
    unsigned lb;
    MLA_LDS char* stage;
  };

  __device__ __forceinline__ Pending prepare(const bf16* __restrict__ base, int row0, int row_end,
                                             MLA_LDS char* stage) const {
    Pending p;
    p.lb = lane_base();
    int rows = row_end - row0;
    rows = rows > KT ? KT : rows;
    rows = rows < 0 ? 0 : rows;  // a tile wholly past row_end reads as zeros
    p.rs = make_rsrc(base + (size_t)row0 * R, (unsigned)(rows * R * 2));
    p.stage = stage;
    return p;
  }

  // Copies c in [C0, C1) of this wave's CPW copies.
  template <int C0, int C1>
  __device__ __forceinline__ void issue_range(const Pending& p) const {
#pragma unroll
    for (int c = C0; c < (C1 < CPW ? C1 : CPW); ++c) {
      const int qi = w + NW * c;
      if (COPIES % NW == 0 || qi < COPIES) {
        const int srow = qi * RPI;
        const unsigned k = (unsigned)((tile_swizzle<R, SW>(srow) << 4) | (srow * R * 2));
        buf2lds16(p.rs, p.lb ^ k, p.stage + qi * 1024);
      }
    }
  }

  // Copy c alone (c < CPW; a constant once the caller is unrolled).
  __device__ __forceinline__ void issue_one(const Pending& p, int c) const {
    const int qi = w + NW * c;
    if (COPIES % NW == 0 || qi < COPIES) {
      const int srow = qi * RPI;
      const unsigned k = (unsigned)((tile_swizzle<R, SW>(srow) << 4) | (srow * R * 2));
      buf2lds16(p.rs, p.lb ^ k, p.stage + qi * 1024);
    }
  }

  // This lane's byte offset for copy qi of any tile (for a wave that keeps
  // it in a register and issues that one copy of every tile).
  __device__ __forceinline__ unsigned offset_of(int qi) const {
    const int srow = qi * RPI;
    return lane_base() ^ (unsigned)((tile_swizzle<R, SW>(srow) << 4) | (srow * R * 2));
  }

  __device__ __forceinline__ void issue(const bf16* __restrict__ base, int row0, int row_end,
                                        MLA_LDS char* stage) const {
    issue_range<0, CPW>(prepare(base, row0, row_end, stage));
  }
};

// q_abs^T for 16 rows: qT[kk] is the score B operand for latent dims
// [32kk, 32kk+32) (slot p <-> dim 32kk + 8kq + p), already multiplied by
// qscale.  qrow points at this lane's query row (DQ values, 16-byte aligned);
// wkT at W_UK^T[h] ([R, DQ]).
template <int DQ, int R>
__device__ __forceinline__ void absorb_rows(const bf16* __restrict__ qrow, const bf16* __restrict__ wkT,
                                            float qscale, int l16, int kq, bf16x8 (&qT)[R / 32]) {
  constexpr int NKQ = (DQ + 31) / 32;
  bf16x8 qb[NKQ];
#pragma unroll
  for (int k = 0; k < NKQ; ++k)
    qb[k] = (32 * k + 8 * kq < DQ) ? *(const bf16x8*)(qrow + 32 * k + 8 * kq) : bf16x8{};
#pragma unroll
  for (int kk = 0; kk < R / 32; ++kk) {
    f32x4 acc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // A row rho loads latent dim 32kk + 8(rho/4) + 4u + rho%4, so C row
      // 4kq + e of this fragment is dim 32kk + 8kq + 4u + e
      const int j = 32 * kk + 8 * (l16 >> 2) + 4 * u + (l16 & 3);
      const bf16* wrow = wkT + (size_t)j * DQ;
      acc[u] = f32x4{};
#pragma unroll
      for (int k = 0; k < NKQ; ++k) {
        const bf16x8 av = (32 * k + 8 * kq < DQ) ? *(const bf16x8*)(wrow + 32 * k + 8 * kq) : bf16x8{};
        acc[u] = mfma16(av, qb[k], acc[u]);
      }
    }
    qT[kk] = pack44(acc[0], acc[1], qscale);
  }
}

// PF > 0: the LDS operands of score k-step kk+PF (value tile t+PF) are read
// while the MFMAs of step kk (tile t) run; two steps ahead measured 7% faster
// than chunked reads on the full-width decode.  With PF = 0, QCH / VCH score
// k-steps / value tiles form one chunk (its reads, then its MFMAs).
template <int R, int QCH = 4, int VCH = 8, int PF = 2>
struct WaveAttn {
  static constexpr int NKK = R / 32;
  static constexpr int NJT = R / 16;
  // The swizzle f(s) only permutes the low 4 bits of a chunk index, so for
  // R >= 128 every operand address is one per-lane base plus a small XOR term
  // and an immediate:
  //  * score operand, row l16, chunk 4kk + kq:  with x = f(l16)
  //      16 ((kq ^ x) & 3) + 64 ((kk & 3) ^ (x >> 2)) + 256 (kk >> 2)
  //  * value operand, row r = 4kq + l16/4, chunk 2t + (l16%4)/2: x = f(r)
  //      16 (((l16%4)/2) ^ (x & 1)) + 32 ((t & 7) ^ (x >> 1)) + 256 (t >> 3)
  // Smaller r keeps one precomputed base per k-step / value tile.
  static constexpr bool XORADDR = (R / 8 >= 16);
  static constexpr int NQB = XORADDR ? 1 : NKK;
  static constexpr int NTB = XORADDR ? 1 : NJT;
  static constexpr int ROWB = R * 2;
  bf16x8 qT[NKK];
  f32x4 oT[NJT];
  float m_run, l_run;
  int qk_base[NQB];
  int tr_base[NTB];
  int qk_x, tr_rx;

  __device__ __forceinline__ void init_addressing(int l16, int kq) {
    const int r = 4 * kq + (l16 >> 2), q = l16 & 3;
    if constexpr (XORADDR) {
      const int x = chunk_swizzle<R>(l16);
      qk_base[0] = l16 * ROWB + (((kq ^ x) & 3) << 4);
      qk_x = x >> 2;
      const int xr = chunk_swizzle<R>(r);
      tr_base[0] = r * ROWB + ((((q >> 1) ^ (xr & 1))) << 4) + (q & 1) * 8;
      tr_rx = xr >> 1;
    } else {
#pragma unroll
      for (int u = 0; u < NQB; ++u) qk_base[u] = tile_off<R>(l16, 4 * u + kq);
#pragma unroll
      for (int u = 0; u < NTB; ++u) tr_base[u] = tile_off<R>(r, 2 * u + (q >> 1)) + (q & 1) * 8;
      qk_x = tr_rx = 0;
    }
  }

  // b / x are per-tile opaque copies of the bases (see scores / update), so
  // the compiler forms each address at its use instead of keeping all of
  // them live across the main loop.
  __device__ __forceinline__ int qk_off(int kk, int b, int x) const {
    if constexpr (XORADDR) {
      return b + (((kk & 3) ^ x) << 6) + (kk >> 2) * 256;
    } else {
      return qk_base[kk];
    }
  }

  __device__ __forceinline__ int tr_off(int t, int b, int x) const {
    if constexpr (XORADDR) {
      return b + (((t & 7) ^ x) << 5) + (t >> 3) * 256;
    } else {
      return tr_base[t];
    }
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int t = 0; t < NJT; ++t) oT[t] = f32x4{};
    m_run = -INFINITY;
    l_run = 0.0f;
  }

  // S^T fragments for keys [0,16) (s0) and [16,32) (s1) of the tile.
  __device__ __forceinline__ void scores(const MLA_LDS char* tile, f32x4& s0, f32x4& s1) const {
    s0 = f32x4{};
    s1 = f32x4{};
    int qb = qk_base[0], qx = qk_x;
    asm volatile("" : "+v"(qb), "+v"(qx));
    constexpr int SP = PF < NKK ? PF : NKK - 1;  // lookahead that exists
    if constexpr (SP > 0) {
      // operands of k-steps kk+1 .. kk+SP are read while k-step kk's MFMAs run
      bf16x8 a[SP + 1][2];
#pragma unroll
      for (int u = 0; u < SP; ++u) {
        const MLA_LDS char* p = tile + qk_off(u, qb, qx);
        a[u][0] = lds_read_b128(p);
        a[u][1] = lds_read_b128(p + 16 * ROWB);
      }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        if (kk + SP < NKK) {
          const MLA_LDS char* p = tile + qk_off(kk + SP, qb, qx);
          a[(kk + SP) % (SP + 1)][0] = lds_read_b128(p);
          a[(kk + SP) % (SP + 1)][1] = lds_read_b128(p + 16 * ROWB);
        }
        __builtin_amdgcn_sched_barrier(0);
        s0 = mfma16(a[kk % (SP + 1)][0], qT[kk], s0);
        s1 = mfma16(a[kk % (SP + 1)][1], qT[kk], s1);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
    constexpr int CH = NKK < QCH ? NKK : QCH;
#pragma unroll
    for (int k0 = 0; k0 < NKK; k0 += CH) {
#pragma unroll
      for (int kk = k0; kk < k0 + CH; ++kk) {
        const MLA_LDS char* p = tile + qk_off(kk, qb, qx);
        s0 = mfma16(lds_read_b128(p), qT[kk], s0);
        s1 = mfma16(lds_read_b128(p + 16 * ROWB), qT[kk], s1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    }
  }

  // Online softmax over one tile's (already masked) log2-domain scores and
  // the value accumulation.  The reference max only moves when a score
  // exceeds it by more than 8, so the O^T rescale is rare and P <= 2^8.
  __device__ __forceinline__ void update(const MLA_LDS char* tile, const f32x4& s0, const f32x4& s1) {
    // value operand: lane i of 16-lane group kq takes latent dim 16t + i and
    // keys {4kq+e} (lo) / {16+4kq+e} (hi); its tr16 source chunk is key row
    // 4kq + i/4 (+16), dims 16t + 4(i%4) .. +3.
    int tb = tr_base[0], tx = tr_rx;
    asm volatile("" : "+v"(tb), "+v"(tx));
    auto rd = [&](int t) {
      const MLA_LDS char* p = tile + tr_off(t, tb, tx);
      return cat4(lds_read_tr16(p), lds_read_tr16(p + 16 * ROWB));
    };
    constexpr int VP = PF < NJT ? PF : NJT - 1;  // lookahead that exists
    // The first value operands do not depend on P: their reads go out before
    // the softmax arithmetic.
    bf16x8 a[VP + 1];
    if constexpr (VP > 0) {
#pragma unroll
      for (int u = 0; u < VP; ++u) a[u] = rd(u);
      __builtin_amdgcn_sched_barrier(0);
    }

    float mx = max8_nn(s0, s1);
    mx = col_max(mx);
    const bool need = mx > m_run + 8.0f;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_new = need ? mx : m_run;
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < NJT; ++t) oT[t] *= alpha;
      m_run = m_new;
    }
    f32x4 p0, p1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p0[e] = fast_exp2(s0[e] - m_run);
      p1[e] = fast_exp2(s1[e] - m_run);
    }
    l_run += (p0[0] + p0[1]) + (p0[2] + p0[3]) + (p1[0] + p1[1]) + (p1[2] + p1[3]);
    const bf16x8 pB = pack44(p0, p1, 1.0f);

    if constexpr (VP > 0) {
      // value tiles t+1 .. t+VP are read while tile t's MFMA runs
#pragma unroll
      for (int t = 0; t < NJT; ++t) {
        if (t + VP < NJT) a[(t + VP) % (VP + 1)] = rd(t + VP);
        __builtin_amdgcn_sched_barrier(0);
        oT[t] = mfma16(a[t % (VP + 1)], pB, oT[t]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      constexpr int CH = NJT < VCH ? NJT : VCH;
#pragma unroll
      for (int t0 = 0; t0 < NJT; t0 += CH) {
#pragma unroll
        for (int t = t0; t < t0 + CH; ++t) oT[t] = mfma16(rd(t), pB, oT[t]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
};

// Epilogue: o^T = W_UV[h] (O^T / l) for 16 rows, gated and stored.  orow
// points at this lane's output row segment for head h (DV values) and grow at
// the matching gate logits; valid = row and head exist.
template <int DV, int R>
__device__ __forceinline__ void project_gate_store(const f32x4 (&oT)[R / 16], float inv_l,
                                                   const bf16* __restrict__ wv, const bf16* __restrict__ grow,
                                                   bf16* __restrict__ orow, bool valid, int l16, int kq) {
  bf16x8 ob[R / 32];
#pragma unroll
  for (int kk = 0; kk < R / 32; ++kk) ob[kk] = pack44(oT[2 * kk], oT[2 * kk + 1], inv_l);
#pragma unroll
  for (int vt = 0; vt < DV / 16; ++vt) {
    const bf16* wrow = wv + (size_t)(16 * vt + l16) * R + 4 * kq;
    f32x4 acc = f32x4{};
#pragma unroll
    for (int kk = 0; kk < R / 32; ++kk) {
      const bf16x4 lo = *(const bf16x4*)(wrow + 32 * kk);
      const bf16x4 hi = *(const bf16x4*)(wrow + 32 * kk + 16);
      acc = mfma16(cat4(lo, hi), ob[kk], acc);
    }
    if (valid) {
      const int v = 16 * vt + 4 * kq;
      const bf16x4 gv = *(const bf16x4*)(grow + v);
      bf16x4 ov;
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[e] = (bf16)(acc[e] * sigmoidf_((float)gv[e]));
      *(bf16x4*)(orow + v) = ov;
    }
  }
}

}  // namespace mla

namespace mla {

// ---------------------------------------------------------------------------
// Wave-pair variant: two waves share 32 query columns (two 16-column groups)
// and split the latent dimension r in halves.  Each latent operand read from
// LDS then feeds two MFMAs (one per column group), halving LDS traffic per
// FLOP, while each wave still holds only a [r/2 x 32] O^T accumulator.  The
// score needs the full r, so the pair adds its two partial S^T tiles through
// LDS once per key tile; both waves then run the same softmax.
// ---------------------------------------------------------------------------

// q_abs^T for two 16-row column groups, latent dims [jbase, jbase + R/2).
template <int DQ, int R>
__device__ __forceinline__ void absorb_pair(const bf16* __restrict__ qrow0, const bf16* __restrict__ qrow1,
                                            const bf16* __restrict__ wkT, int jbase, float qscale, int l16,
                                            int kq, bf16x8 (&qT)[2][R / 64]) {
  constexpr int NKQ = (DQ + 31) / 32;
  bf16x8 qb[2][NKQ];
#pragma unroll
  for (int k = 0; k < NKQ; ++k) {
    const bool ok = 32 * k + 8 * kq < DQ;
    qb[0][k] = ok ? *(const bf16x8*)(qrow0 + 32 * k + 8 * kq) : bf16x8{};
    qb[1][k] = ok ? *(const bf16x8*)(qrow1 + 32 * k + 8 * kq) : bf16x8{};
  }
#pragma unroll
  for (int kk = 0; kk < R / 64; ++kk) {
    f32x4 acc[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // A row rho loads latent dim jbase + 32kk + 8(rho/4) + 4u + rho%4, so C
      // row 4kq + e of this fragment is dim jbase + 32kk + 8kq + 4u + e
      const int j = jbase + 32 * kk + 8 * (l16 >> 2) + 4 * u + (l16 & 3);
      const bf16* wrow = wkT + (size_t)j * DQ;
      acc[0][u] = f32x4{};
      acc[1][u] = f32x4{};
#pragma unroll
      for (int k = 0; k < NKQ; ++k) {
        const bf16x8 av = (32 * k + 8 * kq < DQ) ? *(const bf16x8*)(wrow + 32 * k + 8 * kq) : bf16x8{};
        acc[0][u] = mfma16(av, qb[0][k], acc[0][u]);
        acc[1][u] = mfma16(av, qb[1][k], acc[1][u]);
      }
    }
    qT[0][kk] = pack44(acc[0][0], acc[0][1], qscale);
    qT[1][kk] = pack44(acc[1][0], acc[1][1], qscale);
  }
}

// SPF: score operands of k-step kk+1 are read from LDS while the MFMAs of
// k-step kk run; VPF > 0: value operands run VPF tiles ahead.  Without them,
// QCH / VCH k-steps / value tiles form one chunk (its LDS reads, then its
// MFMAs).  One step of each lookahead measured +2.4% apiece on the full-width
// prefill; two value tiles ahead no longer fit the registers.
template <int R, int QCH = 1, int VCH = 4, bool SPF = true, int VPF = 1>
struct PairAttn {
  static constexpr int RH = R / 2;     // latent dims owned by this wave
  static constexpr int NKK = RH / 32;  // score k-steps
  static constexpr int NJT = RH / 16;  // value tiles
  static constexpr int ROWB = R * 2;
  static_assert(R / 8 >= 16 && NKK % 4 == 0 && NJT % 8 == 0, "pair split needs r >= 256");
  bf16x8 qT[2][NKK];
  f32x4 oT[2][NJT];
  float m_run[2], l_run[2];
  // Operand addresses (latent half folded in): the score operand of k-step kk
  // is qkb[kk & 3] + 256 (kk >> 2), the value operand of tile t is
  // trb[t & 7] + 256 (t >> 3); the immediates fold into the ds_read offsets.
  int qkb[4], trb[8];

  __device__ __forceinline__ void init_addressing(int l16, int kq, int jh) {
    const int x = chunk_swizzle<R>(l16);
    const int qk_base = l16 * ROWB + (((kq ^ x) & 3) << 4) + jh * RH * 2;
#pragma unroll
    for (int u = 0; u < 4; ++u) qkb[u] = qk_base + ((u ^ (x >> 2)) << 6);
    const int r = 4 * kq + (l16 >> 2), q = l16 & 3;
    const int xr = chunk_swizzle<R>(r);
    const int tr_base = r * ROWB + (((q >> 1) ^ (xr & 1)) << 4) + (q & 1) * 8 + jh * RH * 2;
#pragma unroll
    for (int u = 0; u < 8; ++u) trb[u] = tr_base + ((u ^ (xr >> 1)) << 5);
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int t = 0; t < NJT; ++t) oT[c][t] = f32x4{};
      m_run[c] = -INFINITY;
      l_run[c] = 0.0f;
    }
  }

  // Partial S^T over this wave's latent half: s[cg][u] holds keys
  // [16u, 16u+16) of the tile for column group cg.
  // hook(k0) runs after the chunk that starts at k-step k0 (used to spread
  // the next tile's copies over the score products).
  template <typename Hook>
  __device__ __forceinline__ void partial_scores(const MLA_LDS char* tile, f32x4 (&s)[2][2], Hook&& hook) {
#pragma unroll
    for (int c = 0; c < 2; ++c) s[c][0] = s[c][1] = f32x4{};
    // Launder the 4 bases in place each tile: the compiler then cannot hoist
    // 16 base + offset sums out of the loop (they would stay live and
    // spill), and every address is one base plus a ds_read immediate.
    asm volatile("" : "+v"(qkb[0]), "+v"(qkb[1]), "+v"(qkb[2]), "+v"(qkb[3]));
    const int* bq = qkb;
    if constexpr (SPF) {
      // operands of k-step kk+1 are read while the MFMAs of k-step kk run
      bf16x8 a0 = lds_read_b128(tile + bq[0]);
      bf16x8 a1 = lds_read_b128(tile + bq[0] + 16 * ROWB);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        bf16x8 n0 = a0, n1 = a1;
        if (kk + 1 < NKK) {
          const MLA_LDS char* p = tile + bq[(kk + 1) & 3] + ((kk + 1) >> 2) * 256;
          n0 = lds_read_b128(p);
          n1 = lds_read_b128(p + 16 * ROWB);
        }
        __builtin_amdgcn_sched_barrier(0);
        s[0][0] = mfma16(a0, qT[0][kk], s[0][0]);
        s[1][0] = mfma16(a0, qT[1][kk], s[1][0]);
        s[0][1] = mfma16(a1, qT[0][kk], s[0][1]);
        s[1][1] = mfma16(a1, qT[1][kk], s[1][1]);
        __builtin_amdgcn_sched_barrier(0);
        hook(kk);
        a0 = n0;
        a1 = n1;
      }
    } else {
#pragma unroll
    for (int k0 = 0; k0 < NKK; k0 += QCH) {
#pragma unroll
      for (int kk = k0; kk < k0 + QCH; ++kk) {
        const MLA_LDS char* p = tile + bq[kk & 3] + (kk >> 2) * 256;
        const bf16x8 a0 = lds_read_b128(p);
        const bf16x8 a1 = lds_read_b128(p + 16 * ROWB);
        s[0][0] = mfma16(a0, qT[0][kk], s[0][0]);
        s[1][0] = mfma16(a0, qT[1][kk], s[1][0]);
        s[0][1] = mfma16(a1, qT[0][kk], s[0][1]);
        s[1][1] = mfma16(a1, qT[1][kk], s[1][1]);
      }
      __builtin_amdgcn_sched_barrier(0);
      hook(k0);
    }
    }
  }

  // Online softmax of both column groups over the full (masked, log2-domain)
  // scores; returns P^T as the value product's B operands.
  __device__ __forceinline__ void softmax(const f32x4 (&s)[2][2], bf16x8 (&pB)[2]) {
    float mx[2];
    bool need[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const f32x4& a = s[c][0];
      const f32x4& b = s[c][1];
      mx[c] = col_max(max8_nn(a, b));
      need[c] = mx[c] > m_run[c] + 8.0f;
    }
    if (__builtin_amdgcn_ballot_w64(need[0] || need[1])) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float m_new = need[c] ? mx[c] : m_run[c];
        const float alpha = fast_exp2(m_run[c] - m_new);
        l_run[c] *= alpha;
#pragma unroll
        for (int t = 0; t < NJT; ++t) oT[c][t] *= alpha;
        m_run[c] = m_new;
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      f32x4 p0, p1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p0[e] = fast_exp2(s[c][0][e] - m_run[c]);
        p1[e] = fast_exp2(s[c][1][e] - m_run[c]);
      }
      l_run[c] += (p0[0] + p0[1]) + (p0[2] + p0[3]) + (p1[0] + p1[1]) + (p1[2] + p1[3]);
      pB[c] = pack44(p0, p1, 1.0f);
    }
  }

  __device__ __forceinline__ bf16x8 value_operand(const MLA_LDS char* tile, int t) const {
    const MLA_LDS char* p = tile + trb[t & 7] + (t >> 3) * 256;
    return cat4(lds_read_tr16(p), lds_read_tr16(p + 16 * ROWB));
  }

  // Value accumulation of this wave's latent half: O^T += c_tile^T P^T.
  __device__ __forceinline__ void values(const MLA_LDS char* tile, const bf16x8 (&pB)[2]) {
    asm volatile("" : "+v"(trb[0]), "+v"(trb[1]), "+v"(trb[2]), "+v"(trb[3]), "+v"(trb[4]), "+v"(trb[5]),
                      "+v"(trb[6]), "+v"(trb[7]));  // as in partial_scores
    if constexpr (VPF > 0) {
      // operands of value tiles t+1 .. t+VPF are read while the MFMAs of
      // tile t run
      bf16x8 a[VPF + 1];
#pragma unroll
      for (int u = 0; u < VPF; ++u) a[u] = value_operand(tile, u);
#pragma unroll
      for (int t = 0; t < NJT; ++t) {
        if (t + VPF < NJT) a[(t + VPF) % (VPF + 1)] = value_operand(tile, t + VPF);
        __builtin_amdgcn_sched_barrier(0);
        oT[0][t] = mfma16(a[t % (VPF + 1)], pB[0], oT[0][t]);
        oT[1][t] = mfma16(a[t % (VPF + 1)], pB[1], oT[1][t]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int t0 = 0; t0 < NJT; t0 += VCH) {
#pragma unroll
        for (int t = t0; t < t0 + VCH; ++t) {
          const bf16x8 a = value_operand(tile, t);
          oT[0][t] = mfma16(a, pB[0], oT[0][t]);
          oT[1][t] = mfma16(a, pB[1], oT[1][t]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
};

}  // namespace mla
