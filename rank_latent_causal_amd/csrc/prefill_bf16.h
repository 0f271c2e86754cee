// bf16 prefill pieces for the absorbed Gated MLA layer on gfx950: the
// kernel arguments, the varlen block list, the key-tile copies that every
// prefill kernel uses, and the prefill kernel for narrow latents (r = 32; the
// one-wave-per-SIMD kernel of prefill_solo.h covers r >= 256).
//
// mla_prefill_bf16_kernel: one workgroup = 4 waves = 16 query positions x 4
// heads; each wave runs the whole chain of page "Gated MLA（矩阵吸收版）",
// section 完整计算流（四步） steps 2-4 (the same contractions are listed in
// page "符号表", section Einsum 速查) for its rows:
//   prologue  q_abs^T = W_UK[h]^T q^T on MFMA, kept in VGPRs (absorb)
//   main loop causal latent flash attention over 32-key tiles of c
//   epilogue  o^T = W_UV[h] (O^T / l) on MFMA, sigmoid gate, store
// Every latent tile is copied once from global memory straight into LDS
// (LDS-DMA, no register staging) and shared by the four heads: heads are
// folded into the rows that reuse one c tile.  Two LDS stages let the copy
// of tile n+1 overlap tile n.
#pragma once

#include <type_traits>

#include "attn_core.h"

namespace mla {

struct PrefillArgs {
  const bf16* q;     // [B, T, H, DQ]
  const bf16* c;     // [B, S, R]: the T queries are positions S-T .. S-1
  const bf16* wukT;  // [H, R, DQ]  (W_UK transposed per head, in the workspace)
  const bf16* wuv;   // [H, DV, R]
  const bf16* gate;  // [B, T, H*DV]
  bf16* out;         // [B, T, H*DV]
  int B, T, H;
  int S;             // latent rows per sequence (S >= T; S - T cached prefix positions)
  float qscale;      // softmax scale * log2(e), folded into q_abs
  int ntb;           // ceil(T / kPrefillRows) query blocks
  int nhg;           // ceil(H / 4) head groups
  int xcd_remap;     // 1: head group hg runs on XCD hg % 8 (weights stay in its L2)
  // if set (r >= 256 kernel, not varlen): workgroups take work items in the
  // order they start from this counter, which is zero at launch (the W_UK
  // transpose clears it), instead of from blockIdx
  unsigned* queue;
  // paged latent (the kernels' PAGED instantiations): c is a pool of
  // num_pages pages of 2^page_shift rows (at least the 32-row key tile);
  // row u of sequence b is page block_table[b, u >> page_shift], slot
  // u & (2^page_shift - 1).  A page index outside [0, num_pages) reads as
  // zero rows.
  const int* block_table;  // [B, max_pages]
  int page_shift, max_pages, num_pages;
  // training: the natural-log log-sum-exp of each row's scaled scores,
  // [B, H, T] (written when non-null; the backward recomputes P from it)
  float* lse;
  // varlen (the VARLEN instantiations, always paged): query blocks come from
  // a list built by mla_varlen_prepare; sequence b owns packed query rows
  // seq[b].x .. seq[b].x + seq[b].y - 1 and seq[b].z cache rows
  const int4* seq;      // [B] {first query row, T_b, S_b, 0}
  const int2* blocks;   // [max blocks] {b, query block}
  const int* nblocks;   // number of valid blocks
};

// One workgroup: sanitises the varlen description (query ranges inside
// [0, Nq), cache lengths inside [0, max_rows)) and lists the query blocks of
// BR rows, each sequence's heaviest (last) block first.  At most max_blocks
// entries are written.
__global__ void __launch_bounds__(256) mla_varlen_prepare(const int* __restrict__ cu_q,
                                                          const int* __restrict__ seq_lens, int B, int Nq,
                                                          int max_rows, int BR, int max_blocks, int4* __restrict__ seq,
                                                          int2* __restrict__ blocks, int* __restrict__ nblocks) {
  __shared__ int wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int carry = 0;
  for (int base = 0; base < B; base += 256) {
    const int b = base + tid;
    int nb = 0, q0 = 0, T = 0, S = 0;
    if (b < B) {
      q0 = min(max(cu_q[b], 0), Nq);
      T = max(0, min(max(cu_q[b + 1], 0), Nq) - q0);
      S = min(max(seq_lens[b], 0), max_rows);
      nb = (T + BR - 1) / BR;
      seq[b] = make_int4(q0, T, S, 0);
    }
    int incl = nb;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int off = carry + incl - nb;
    for (int u = 0; u < w; ++u) off += wsum[u];
    for (int k = 0; k < nb; ++k)
      if (off + k < max_blocks) blocks[off + k] = make_int2(b, nb - 1 - k);
    carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  if (tid == 0) *nblocks = min(carry, max_blocks);
}

// Issues the copies of key tile j (rows 32j .. 32j+31 of sequence b) into an
// LDS stage: from the contiguous latent [B, S, R], or through the block table.
// prepare_key_tile forms the descriptor and offsets only; the copies then go
// out with copier.issue_range / issue_one.  With real = false the descriptor
// covers no bytes (the copies write zero rows), so callers can issue a tile's
// copies without a branch; the block-table lookup then reads entry 0.
template <bool PAGED, int R, int NW, int SW>
__device__ __forceinline__ typename TileCopier<R, NW, SW>::Pending prepare_key_tile(
    const TileCopier<R, NW, SW>& copier, const PrefillArgs& a, int b, int S, int j, MLA_LDS char* stage,
    bool real = true, bool with_lane_base = true) {
  constexpr int KT = LatentTile<R>::KT;
  if constexpr (PAGED) {
    const int pos = real ? j * KT : 0;
    int pg = sload_i32(a.block_table + (size_t)b * a.max_pages + (pos >> a.page_shift));
    int valid = real ? min(S - pos, KT) : 0;
    if ((unsigned)pg >= (unsigned)a.num_pages) {
      pg = 0;
      valid = 0;
    }
    const size_t row = ((size_t)pg << a.page_shift) + (pos & ((1 << a.page_shift) - 1));
    return copier.prepare(a.c + row * R, 0, valid, stage, with_lane_base);
  } else {
    return copier.prepare(a.c + (size_t)b * S * R, j * KT, real ? S : 0, stage, with_lane_base);
  }
}

template <bool PAGED, int R, int NW, int SW>
__device__ __forceinline__ void issue_key_tile(const TileCopier<R, NW, SW>& copier, const PrefillArgs& a, int b, int S,
                                               int j, MLA_LDS char* stage, bool real = true) {
  copier.template issue_range<0, TileCopier<R, NW, SW>::CPW>(
      prepare_key_tile<PAGED>(copier, a, b, S, j, stage, real));
}

// waves per workgroup: 4 heads x (kPrefillWaves / 4) blocks of 16 positions
constexpr int kPrefillWaves = 4;
constexpr int kPrefillRows = 16 * (kPrefillWaves / 4);  // query positions per workgroup

template <int DQ, int DV, int R, bool PAGED = false, bool VARLEN = false>
__global__ void __launch_bounds__(64 * kPrefillWaves)
__attribute__((amdgpu_waves_per_eu(2, 2)))
mla_prefill_bf16_kernel(PrefillArgs a) {
  using LT = LatentTile<R>;
  constexpr int NS = 2;
  constexpr int LPW = copies_per_wave<R>(kPrefillWaves);
  static_assert(LT::COPIES % kPrefillWaves == 0 || LT::COPIES < kPrefillWaves, "copy split");
  static_assert(DQ % 16 == 0 && DV % 16 == 0 && R % 32 == 0, "shape");
  __shared__ __attribute__((aligned(1024))) char smem_raw[NS * LT::BYTES];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;

  // ---- work item: heaviest query blocks first
  const int x = blockIdx.x;
  int tb, b, hg;
  if constexpr (VARLEN) {
    hg = x % a.nhg;
    const int i = x / a.nhg;
    if (i >= __builtin_amdgcn_readfirstlane(*a.nblocks)) return;  // the whole workgroup
    const int2 e = a.blocks[i];
    b = __builtin_amdgcn_readfirstlane(e.x);
    tb = __builtin_amdgcn_readfirstlane(e.y);
  } else if (a.xcd_remap) {
    // gridDim.x = 8 * per; XCD x % 8 owns head groups hg = x % 8 (mod 8)
    const int xcd = x & 7, pos = x >> 3, nh8 = a.nhg >> 3;
    hg = (pos % nh8) * 8 + xcd;
    const int rest = pos / nh8;
    b = rest % a.B;
    tb = a.ntb - 1 - rest / a.B;
  } else {
    hg = x % a.nhg;
    const int rest = x / a.nhg;
    b = rest % a.B;
    tb = a.ntb - 1 - rest / a.B;
  }

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, kq = lane >> 4;
  const int hw = w & 3, th = w >> 2;  // head in group, 16-row block
  const int h = hg * 4 + hw;
  const bool hvalid = h < a.H;
  const int hc = hvalid ? h : a.H - 1;
  const int H = a.H;
  int T = a.T, S = a.S;
  size_t qr0 = (size_t)b * a.T;  // packed row of query 0 of sequence b
  if constexpr (VARLEN) {
    const int4 sq = a.seq[b];
    qr0 = (size_t)__builtin_amdgcn_readfirstlane(sq.x);
    T = __builtin_amdgcn_readfirstlane(sq.y);
    S = __builtin_amdgcn_readfirstlane(sq.z);
  }
  const int t0 = tb * kPrefillRows;
  const int tw = t0 + 16 * th;  // first row of this wave
  const int t = tw + l16;       // this lane's query row
  const bool tvalid = t < T;
  const int tc = tvalid ? t : T - 1;
  const int P = S - T;  // query t sits at position P + t

  const int ntiles = (P + min(t0 + kPrefillRows, T) + LT::KT - 1) / LT::KT;

  // stream the first latent tile while the absorb prologue runs
  TileCopier<R, kPrefillWaves> copier;
  copier.init(w, lane);
  issue_key_tile<PAGED>(copier, a, b, S, 0, smem);

  WaveAttn<R> st;
  absorb_rows<DQ, R>(a.q + ((qr0 + tc) * H + hc) * DQ, a.wukT + (size_t)hc * R * DQ, a.qscale,
                     l16, kq, st.qT);
  st.reset();
  st.init_addressing(l16, kq);

  for (int it = 0; it < ntiles; ++it) {
    if (it + 1 < ntiles) {
      issue_key_tile<PAGED>(copier, a, b, S, it + 1, smem + ((it + 1) & 1) * LT::BYTES);
      wait_vmcnt<LPW>();
    } else {
      wait_vmcnt<0>();
    }
    wg_barrier();
    const MLA_LDS char* tile = smem + (it & 1) * LT::BYTES;
    const int s0 = it * LT::KT;
    f32x4 sa, sb;
    st.scores(tile, sa, sb);
    if (s0 + LT::KT - 1 > P + tw) {  // causal mask (also hides keys past S)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (s0 + 4 * kq + e > P + t) sa[e] = -INFINITY;
        if (s0 + 16 + 4 * kq + e > P + t) sb[e] = -INFINITY;
      }
    }
    st.update(tile, sa, sb);
    wg_barrier();  // this stage is refilled by the next iteration
  }

  const float l_tot = col_sum(st.l_run);
  const float inv_l = 1.0f / l_tot;
  if (a.lse && kq == 0 && tvalid && hvalid)
    a.lse[((size_t)b * H + h) * T + t] = (st.m_run + __builtin_log2f(l_tot)) * 0.69314718055994531f;
  const size_t orow = (qr0 + tc) * (size_t)H * DV + (size_t)hc * DV;
  project_gate_store<DV, R>(st.oT, inv_l, a.wuv + (size_t)hc * DV * R, a.gate + orow, a.out + orow,
                            tvalid && hvalid, l16, kq);
}

}  // namespace mla
