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
                                             MLA_LDS char* stage, bool with_lane_base = true) const {
    Pending p;
    p.lb = with_lane_base ? lane_base() : 0u;  // without: the caller keeps the copy offsets
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
