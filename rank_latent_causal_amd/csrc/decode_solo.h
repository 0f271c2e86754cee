// One-wave-per-SIMD bf16 split decode for the absorbed Gated MLA layer at
// r = 512 on gfx950.  The cache holds only the latent c (page "Gated MLA
// （矩阵吸收版）", section 低秩压缩 and the KV-cache table of section
// 形状与参数对比), so decode streams c once from HBM and scores every head
// against it; this kernel is the streaming part of that step.
//
// Work split.  Each sequence's cache rows are cut into 32-row tiles of its
// own (the last one partial), so a tile never holds two sequences; the tiles
// of all sequences form one virtual sequence of NT tiles (prefix sums cu_t),
// and workgroup k takes tiles [rt[k], rt[k + 1]), ranges of equal cost where
// a sequence start costs several tiles (mla_paged_prepare).  A
// workgroup is 4 waves, one per SIMD; wave w owns heads 32w .. 32w + 31 over
// the whole latent width, so per tile it runs, on v_mfma_f32_32x32x16_bf16
// (transposed products, one head column per lane pair):
//   S^T  = c_tile . q_abs^T          32 keys x 32 heads, fp32
//   P    = exp2(S - m), online softmax
//   O^T += c_tile^T . P^T             [r x 32] fp32 in accumulation registers
// Every tile is copied once into LDS (LDS-DMA, four stages) and read by
// every computing wave; the score products of tile i+1 run under the
// softmax and between the value products of tile i, as in the
// one-wave-per-SIMD prefill.  With one wave per SIMD, a wave issues at most
// one instruction every few cycles, so the loop is bounded by its own
// instruction count as much as by the matrix unit: at H <= 96 the wave
// without heads takes nearly all tile copies off the computing waves.
//
// Where a sequence ends inside the range, the wave stores that piece's
// unnormalised partial (m and l in fp32, O in bf16, slot k + i for sequence
// i), loads the next sequence's q_abs and starts over with O = 0; the
// partials are merged by mla_decode_merge, whose ranges are in tile units
// here.
#pragma once

#include "decode_bf16.h"
#include "solo_core.h"

namespace mla {

constexpr int kDecodeSoloWaves = 4;
constexpr int kDecodeSoloHeads = 32 * kDecodeSoloWaves;  // heads per workgroup (the largest H)
constexpr int kDecodeSoloStages = 5;  // 160 KiB of LDS
// Cost of a sequence start in tiles, for cutting the ranges: the workgroup
// stores the finished piece's partial (scattered 8-byte stores) and loads
// the next query, about as long as eight tiles.
constexpr int kDecodeSwitchTiles = 8;

struct DecodeSoloArgs {
  const bf16* qabs;         // [B, H, R], scaled by scale * log2(e)
  const bf16* cache;        // packed: [N, R]; paged: [num_pages, page_size, R]
  const int* cu;            // packed: [B + 1] first row of each sequence (the caller's cu_seqlens)
  const int* block_table;   // paged: [B, max_pages]
  const int* lens;          // [B] lengths clamped to [1, rows available] (mla_paged_prepare)
  const int* cu_t;          // [B + 2] tile prefix sums, then the range count (mla_paged_prepare)
  const int* rt;            // [G + 1] first tile of each range (mla_paged_prepare)
  bf16* part_o;             // [(G + B), H, R]  unnormalised O, bf16
  float* part_ml;           // [(G + B), H, 2]
  int B, H;
  int N;                                 // packed: cache rows (< 2^31); no copy reads at or past row N
  int page_shift, max_pages, num_pages;  // paged: pages of 2^page_shift rows
};

// Where the tiles of the range live: sequence, its tile span [t0, t1), its
// length and (packed) first row.  Scalar state, advanced one sequence at a
// time with scalar loads; it never walks past the last sequence.
struct SeqCursor {
  int seq, t0, t1, len, start;
  int page, pg;  // paged: block-table entry looked up last (page -1: none)

  template <bool PAGED>
  __device__ __forceinline__ void init(const DecodeSoloArgs& a, int i) {
    seq = i;
    t0 = sload_i32(a.cu_t + i);
    t1 = sload_i32(a.cu_t + i + 1);
    len = sload_i32(a.lens + i);
    start = PAGED ? 0 : sload_i32(a.cu + i);
    page = -1;
    pg = 0;
  }
  template <bool PAGED>
  __device__ __forceinline__ void seek(const DecodeSoloArgs& a, int t) {
    while (t >= t1 && seq + 1 < a.B) {
      ++seq;
      t0 = t1;
      t1 = sload_i32(a.cu_t + seq + 1);
      len = sload_i32(a.lens + seq);
      if constexpr (!PAGED) start = sload_i32(a.cu + seq);
      page = -1;
    }
  }
};

// v-th 4-element group of an accumulation-register block, read in assembly
// (a compiler read of O^T inside the loop would copy the block through VGPRs)
__device__ __forceinline__ f32x4 read_acc4(const f32x16& c, int g) {
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r[e]) : "a"(c[4 * g + e]));
  return r;
}

// Copies and barriers.  Tile x goes into stage x % 5.  One barrier per step,
// in the middle of step s's value products, publishes tile s+2 (every wave's
// copies of it have landed) and shows that every wave has finished step s-1,
// whose tile s-1 held the stage that tile s+4 then takes: a copy goes out two
// steps before it is needed, and the next step's first operands are read
// before the step ends, so the matrix unit does not wait for a barrier at
// the step boundary.
// SPARE (H <= 96): wave 3 has no heads and issues copies 0..28 of every tile
// right after the barrier (a wave keeps at most 63 loads in flight, and two
// tiles' worth are); waves 0..2 issue copy 29 + w of every tile, so each
// step gives them the same work and none holds up the barrier.
// Otherwise (96 < H <= 128) every wave computes and issues copies w, w + 4,
// .. of each tile, one per value product after the barrier.
template <int R, bool PAGED, bool SPARE>
__global__ void __launch_bounds__(64 * kDecodeSoloWaves)
__attribute__((amdgpu_waves_per_eu(1, 1)))
mla_decode_solo(DecodeSoloArgs a) {
  using LT = LatentTile<R>;
  using SA = SoloAttn<R>;
  constexpr int NS = kDecodeSoloStages;
  constexpr int NW = kDecodeSoloWaves;
  constexpr int KT = LT::KT;
  constexpr int NCP = LT::COPIES;            // 1 KiB copies per tile
  constexpr int CPW = SPARE ? 1 : NCP / NW;  // copies per computing wave and tile
  constexpr int NCC = NCP - 3;               // SPARE: the copier's copies per tile
  using Copier = std::conditional_t<SPARE, TileCopier<R, 1, 1>, TileCopier<R, NW, 1>>;
  constexpr int NKK = SA::NKK, NLB = SA::NLB;
  constexpr int EPK = 16 / (NKK / 2);  // exponentials per phase-A product
  constexpr int RING = 4;              // operand registers in flight (two products of lookahead)
  constexpr int NB = 2 * NLB;          // value products per tile
  constexpr int BAR = NKK / 2 + 6;     // phase-B slot of the barrier
  static_assert(R == 512 && NS == 5 && NCP % NW == 0 && 2 * NCC < 64, "decode layout");
  static_assert(NB % RING == 0 && NKK % RING == 0 && BAR + CPW < NB, "operand rings and slots");
  __shared__ __attribute__((aligned(1024))) char smem_raw[NS * LT::BYTES];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;

  const int k = blockIdx.x;
  const int B = a.B, H = a.H;
  const int lo = sload_i32(a.rt + k), hi = sload_i32(a.rt + k + 1);
  if (lo >= hi) return;  // an empty range: the whole workgroup leaves
  const int ntiles = hi - lo;

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const bool compute = 32 * w < H && (!SPARE || w < NW - 1);  // wave-uniform
  const int h = 32 * w + l32;
  const int hc = h < H ? h : H - 1;

  // the sequence of tile lo: the largest i with cu_t[i] <= lo
  int i0;
  {
    int l = 0, r = B - 1;
    while (l < r) {
      const int mid = (l + r + 1) >> 1;
      if (sload_i32(a.cu_t + mid) <= lo) l = mid; else r = mid - 1;
    }
    i0 = l;
  }

  // ---- tile copies.  A tile past the range is copied with an empty
  // descriptor (zero rows), so the pipeline needs no branch around its
  // copies.  The descriptor arithmetic is 32-bit and scalar (the host keeps
  // the cache below 2^31 rows).
  Copier copier;
  copier.init(SPARE ? 0 : w, lane);
  SeqCursor cc;
  cc.init<PAGED>(a, i0);
  auto tile_src = [&](int x, int& valid) {
    valid = 0;
    const bf16* src = a.cache;
    if (x < ntiles) {
      const int t = lo + x;
      cc.seek<PAGED>(a, t);
      const int dt = t - cc.t0;  // tile of its sequence (below 2^26 for valid lengths)
      const int pos = dt < (1 << 26) ? dt * KT : 0;
      valid = dt < (1 << 26) ? min(cc.len - pos, KT) : 0;
      if constexpr (PAGED) {
        const int pidx = pos >> a.page_shift;
        if (pidx != cc.page && pidx < a.max_pages) {
          cc.page = pidx;
          cc.pg = sload_i32(a.block_table + (size_t)cc.seq * a.max_pages + pidx);
        }
        if (pidx != cc.page || (unsigned)cc.pg >= (unsigned)a.num_pages) valid = 0;
        const size_t row = ((size_t)(valid > 0 ? cc.pg : 0) << a.page_shift) + (pos & ((1 << a.page_shift) - 1));
        src = a.cache + row * R;
      } else {
        // rows start + pos .., clipped at N; a start outside [0, N) reads nothing
        const int rem = (unsigned)cc.start < (unsigned)a.N ? a.N - cc.start : 0;
        valid = pos < rem ? min(valid, rem - pos) : 0;
        src = a.cache + (size_t)(valid > 0 ? cc.start + pos : 0) * R;
      }
    }
    return src;
  };
  auto prepare_tile = [&](int x) {
    int valid;
    const bf16* src = tile_src(x, valid);
    return copier.prepare(src, 0, valid, smem + (x % NS) * LT::BYTES);
  };
  // SPARE: waves 0..2 issue copy NCC + w of every tile, at a lane offset
  // formed once
  const int own_qi = NCC + (w < 3 ? w : 0);
  const unsigned own_off = copier.offset_of(own_qi);
  auto issue_own = [&](int x) {
    int valid;
    const bf16* src = tile_src(x, valid);
    buf2lds16(make_rsrc(src, (unsigned)(valid * R * 2)), own_off, smem + (x % NS) * LT::BYTES + own_qi * 1024);
  };

  if constexpr (SPARE) {
    if (w == NW - 1) {
      // ---- the copier: copies 0 .. NCC-1 of every tile, two tiles in flight
      copier.template issue_range<0, NCC>(prepare_tile(0));
      copier.template issue_range<0, NCC>(prepare_tile(1));
      wait_vmcnt<NCC>();  // tile 0
      copier.template issue_range<0, NCC>(prepare_tile(2));
      wait_vmcnt<NCC>();  // tile 1
      copier.template issue_range<0, NCC>(prepare_tile(3));
      wg_barrier();  // tiles 0 and 1 visible
      for (int s = 0; s < ntiles; ++s) {
        wait_vmcnt<NCC>();  // tile s+2
        wg_barrier();       // tile s+2 visible; step s-1 done everywhere
        copier.template issue_range<0, NCC>(prepare_tile(s + 4));
      }
      wait_vmcnt<0>();
      return;
    }
  }

  if (!compute) {
    // ---- a wave without heads: barriers, and (SPARE) its share of the
    // last copies
    if constexpr (SPARE) {
#pragma unroll
      for (int p = 0; p < NS - 1; ++p) issue_own(p);
    } else {
#pragma unroll
      for (int p = 0; p < NS - 1; ++p) copier.template issue_range<0, CPW>(prepare_tile(p));
    }
    wait_vmcnt<2 * CPW>();  // tiles 0 and 1
    wg_barrier();
    for (int s = 0; s < ntiles; ++s) {
      wait_vmcnt<CPW>();  // tile s+2
      wg_barrier();
      if constexpr (SPARE) issue_own(s + 4);
      else copier.template issue_range<0, CPW>(prepare_tile(s + 4));
    }
    wait_vmcnt<0>();
    return;
  }

  // ---- q_abs^T of the first sequence, then this wave's first copies
  bf16x8 qT[NKK];
  auto load_q = [&](int seq) {
    const bf16* src = a.qabs + ((size_t)seq * H + hc) * R + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qT[kk] = *(const bf16x8*)(src + 16 * kk);
  };
  load_q(i0);
  wait_vmcnt<0>();
  if constexpr (SPARE) {
#pragma unroll
    for (int p = 0; p < NS - 1; ++p) issue_own(p);
  } else {
#pragma unroll
    for (int p = 0; p < NS - 1; ++p) copier.template issue_range<0, CPW>(prepare_tile(p));
  }
  wait_vmcnt<2 * CPW>();  // this wave's copies of tiles 0 and 1

  SA sa;
  sa.init_addressing(lane);
  f32x16 oT[NLB];
  {
    bf16x8 z = bf16x8{};
    asm volatile("" : "+v"(z));
    operand_gap();
#pragma unroll
    for (int u = 0; u < NLB; ++u) zero_a(oT[u], z);
  }
  float m_run, l_run = 0.0f;

  // keys at or past nvalid (rows past the sequence's end) are masked; the
  // key of register r is 8 (r / 4) + 4 (l / 32) + r % 4
  auto mask = [&](f32x16& sv, int nvalid) __attribute__((always_inline)) {
    if (nvalid < KT) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + 4 * hh + (r & 3) >= nvalid) sv[r] = -INFINITY;
    }
  };
  auto tile_at = [&](int x) { return smem + (x % NS) * LT::BYTES; };

  // ---- the sequence piece at hand: local index of the sequence's last tile
  // (may lie past the range) and its valid keys; the next sequence's first
  // tile (its valid keys) and last tile
  int cur = i0, cur_last, cur_nv, next_nv, next_last;
  auto enter_seq = [&](int i) {
    const int t0 = sload_i32(a.cu_t + i), t1 = sload_i32(a.cu_t + i + 1);
    const int len = sload_i32(a.lens + i);
    cur = i;
    cur_last = t1 - 1 - lo;
    cur_nv = len - 32 * (t1 - 1 - t0);
    next_nv = i + 1 < B ? min(sload_i32(a.lens + i + 1), KT) : KT;
    next_last = i + 1 < B ? sload_i32(a.cu_t + i + 2) - 1 - lo : ntiles;
  };
  enter_seq(i0);
  auto nvalid_of = [&](int x) { return x < cur_last ? KT : x == cur_last ? cur_nv : next_nv; };

  // ---- tiles 0 and 1 visible: scores of tile 0, first operands of step 0
  wg_barrier();
  bf16x8 ao[RING], av[RING];
  f32x16 sc;
  {
    ao[0] = sa.score_operand(smem, 0);
    ao[1] = sa.score_operand(smem, 1);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (kk + 2 < NKK) ao[(kk + 2) % RING] = sa.score_operand(smem, kk + 2);
      __builtin_amdgcn_sched_barrier(0);
      if (kk == 0) mfma32v_first(sc, ao[0], qT[0]);
      else mfma32v(sc, ao[kk % RING], qT[kk]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  ao[0] = sa.score_operand(tile_at(1), 0);
  ao[1] = sa.score_operand(tile_at(1), 1);
  av[0] = sa.value_operand(smem, 0);
  av[1] = sa.value_operand(smem, 1);
  settle_v(sc);
  mask(sc, nvalid_of(0));
  float mx;
  {
    const float m0 = max3_nn(sc[0], sc[1], sc[2]), m1 = max3_nn(sc[3], sc[4], sc[5]);
    const float m2 = max3_nn(sc[6], sc[7], sc[8]), m3 = max3_nn(sc[9], sc[10], sc[11]);
    const float m4 = max3_nn(sc[12], sc[13], sc[14]);
    mx = xhalf_max(max3_nn(max3_nn(m0, m1, m2), max3_nn(m3, m4, sc[15]), -INFINITY));
  }
  m_run = mx;

  // The reference max moves only when a score exceeds it by more than 8 (so
  // P <= 2^8): the O^T rescale is rare.
  auto maybe_rescale = [&]() __attribute__((always_inline)) {
    const bool need = mx > m_run + 8.0f;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_new = need ? mx : m_run;
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
      wait_states_24();  // the last value products have written O^T
#pragma unroll
      for (int u = 0; u < NLB; ++u) scale_acc(oT[u], alpha);
      wait_states_24();  // the rescaled O^T feeds the next value products
      m_run = m_new;
    }
  };


  // One step: value products of tile `it` and score products of tile it+1.
  // On entry sc holds the masked scores of tile it and mx their column
  // maxima, ao[0..1] the first score operands of tile it+1 and av[0..1] the
  // first value operands of tile it; on exit, the same for it+1.
  // With next_q >= 0, tile it+2 starts sequence next_q: its q_abs is loaded
  // once the last score product of this step has read q_abs, and waited for
  // at the end of the step.
  auto step = [&](int it, int nvalid1, int next_q) __attribute__((always_inline)) {
    const MLA_LDS char* tile = tile_at(it);
    const MLA_LDS char* tnext = tile_at(it + 1);
    const MLA_LDS char* tnext2 = tile_at(it + 2);
    maybe_rescale();

    // phase A: score products of tile it+1 (k-blocks 0 .. NKK/2-1) under the
    // exponentials of tile it
    f32x16 sn;
#pragma unroll
    for (int kk = 0; kk < NKK / 2; ++kk) {
      ao[(kk + 2) % RING] = sa.score_operand(tnext, kk + 2);
      __builtin_amdgcn_sched_barrier(0);
      if (kk == 0) mfma32v_first(sn, ao[0], qT[0]);
      else mfma32v(sn, ao[kk % RING], qT[kk]);
#pragma unroll
      for (int e = EPK * kk; e < EPK * (kk + 1); ++e) sc[e] = fast_exp2(sc[e] - m_run);
      __builtin_amdgcn_sched_barrier(0);
    }
    // P is packed by VALU instructions: each half is materialised where it is
    // formed and read by a product at least two wait states later
    bf16x8 pB0 = pack8(sc, 0, 1.0f), pB1;
    asm volatile("" : "+v"(pB0));
    operand_gap();
    typename Copier::Pending pend{};
    float m0 = 0.0f, m1 = 0.0f;
    // phase B: value products of tile it in key-block-major order (n = NLB kb
    // + t), the first NKK/2 each followed by one of the remaining score
    // products of tile it+1; the softmax sums, then the mask and column
    // maxima of tile it+1, one piece per product; the barrier at slot BAR;
    // the first operands of the next step at the end
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      if (n + 2 < NB) av[(n + 2) % RING] = sa.value_operand(tile, n + 2);
      else av[(n + 2) % RING] = sa.value_operand(tnext, n + 2 - NB);
      __builtin_amdgcn_sched_barrier(0);
      mfma32a(oT[n % NLB], av[n % RING], n < NLB ? pB0 : pB1);
      __builtin_amdgcn_sched_barrier(0);
      if (n < NKK / 2) {
        const int kk = NKK / 2 + n;
        if (kk + 2 < NKK) ao[(kk + 2) % RING] = sa.score_operand(tnext, kk + 2);
        mfma32v(sn, ao[kk % RING], qT[kk]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (n == 0) {
        pB1 = pack8(sc, 8, 1.0f);
        asm volatile("" : "+v"(pB1));
        __builtin_amdgcn_sched_barrier(0);
      }
      if (n == 1) {
        l_run = sum8_bf16(pB1, sum8_bf16(pB0, l_run));
        __builtin_amdgcn_sched_barrier(0);
      }
      if (n == NKK / 2 + 1) {
        settle_v(sn);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (n == NKK / 2 + 2) {
        mask(sn, nvalid1);
        m0 = max3_nn(max3_nn(sn[0], sn[1], sn[2]), max3_nn(sn[3], sn[4], sn[5]), max3_nn(sn[6], sn[7], -INFINITY));
        __builtin_amdgcn_sched_barrier(0);
      }
      if (n == NKK / 2 + 3) {
        m1 = max3_nn(max3_nn(sn[8], sn[9], sn[10]), max3_nn(sn[11], sn[12], sn[13]), max3_nn(sn[14], sn[15], m0));
        __builtin_amdgcn_sched_barrier(0);
      }
      if (n == NKK / 2 + 4) {
        mx = xhalf_max(m1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (n == BAR - 1) {
        if (next_q >= 0) load_q(next_q);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (n == BAR) {
        // this wave's copies of tile it+2 landed (those of tile it+3 and the
        // q_abs loads just issued are younger); then tile it+2 is visible and
        // every wave is done with step it-1 (tile it-1's stage is free)
        if (next_q >= 0) wait_vmcnt<CPW + NKK>();
        else wait_vmcnt<CPW>();
        wg_barrier();
        if constexpr (SPARE) issue_own(it + 4);
        else pend = prepare_tile(it + 4);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (!SPARE) {
        if (n > BAR && n <= BAR + CPW) {
          copier.issue_one(pend, n - BAR - 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (n == NB - 4 || n == NB - 3) {
        // first score operands of tile it+2 for the next step
        ao[n - (NB - 4)] = sa.score_operand(tnext2, n - (NB - 4));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    sc = sn;
    if (next_q >= 0) wait_vmcnt<0>();  // no load stays pending across the loop's back edge
  };

  // The unnormalised partial of the current sequence piece: O^T in bf16
  // (lane column h, latent dims 32 u + 8 g + 4 (l / 32) + 0..3 of register
  // group g of block u), then m and l.
  auto emit = [&](int seq) {
    wait_states_24();  // the last value products have written O^T
    const float l_tot = xhalf_sum(l_run);
    if (h < H) {
      const size_t slot = (size_t)k + seq;
      bf16* dst = a.part_o + (slot * H + h) * R + 4 * hh;
#pragma unroll
      for (int u = 0; u < NLB; ++u)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v = read_acc4(oT[u], g);
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
          *(bf16x4*)(dst + 32 * u + 8 * g) = o;
        }
      if (hh == 0) {
        a.part_ml[(slot * H + h) * 2 + 0] = m_run;
        a.part_ml[(slot * H + h) * 2 + 1] = l_tot;
      }
    }
  };

  for (int it = 0; it < ntiles; ++it) {
    // tile it+1 starts the next sequence: it is scored against that
    // sequence's q_abs, loaded during the previous step (here only if tile
    // it+1 is the range's second tile)
    const bool new1 = it + 1 < ntiles && it == cur_last && cur + 1 < B;
    // tile it+2 starts sequence cur+1, or (tile it+1 being cur+1's only
    // tile) cur+2
    int q2 = -1;
    if (it + 2 < ntiles) {
      if (it + 1 == cur_last && cur + 1 < B) q2 = cur + 1;
      else if (new1 && it + 1 == next_last && cur + 2 < B) q2 = cur + 2;
    }
    if (new1 && it == 0) {
      load_q(cur + 1);
      wait_vmcnt<0>();
    }
    step(it, nvalid_of(it + 1), q2);
    if (new1) {
      // the piece of sequence `cur` is complete: store it, then start the
      // next one from O = 0, l = 0 and the maxima of its first tile
      emit(cur);
      enter_seq(cur + 1);
      {
        bf16x8 z = bf16x8{};
        asm volatile("" : "+v"(z));
        operand_gap();
#pragma unroll
        for (int u = 0; u < NLB; ++u) zero_a(oT[u], z);
      }
      l_run = 0.0f;
      m_run = mx;
    }
  }
  // this wave's zero-row copies past the range still write the stages: they
  // must land before the workgroup's LDS is released.  The wait comes before
  // the last partial's stores, which the wave leaves in flight (the counter
  // covers stores too, and waiting for them held every workgroup's end)
  wait_vmcnt<0>();
  emit(cur);
}

}  // namespace mla
