// Single-wave-per-SIMD bf16 prefill for the absorbed Gated MLA layer (r >= 256)
// on gfx950.
//
// One workgroup = 4 waves = 128 query positions of one head; each wave owns
// 32 of the positions over the WHOLE latent width r, so the score of page
// "Gated MLA（矩阵吸收版）", section 完整计算流（四步） step 2 is complete
// inside the wave: no partial scores are exchanged.  Per 32-key tile of c the
// wave runs, on v_mfma_f32_32x32x16_bf16 (transposed products, each lane owns
// one query column):
//   S^T  = c_tile . q_abs^T          32x32 fp32 (VGPRs)
//   P    = exp2(S - m), online softmax (lanes l and l^32 share a column)
//   O^T += c_tile^T . P^T             [r x 32] fp32 (accumulation registers)
// The accumulator O^T takes r/2 = 256 registers per lane at r = 512, so the
// kernel runs one wave per SIMD with the accumulation register file for O^T
// and the architectural file for q_abs^T (r/4 registers) and the pipeline.
// With a single wave per SIMD, latency is hidden inside the wave: the score
// products of tile i+1 are issued under the softmax of tile i and between the
// value products of tile i, so the matrix pipe has independent work while the
// softmax arithmetic and the LDS reads are in flight.
// Every c tile is copied once per workgroup into LDS (LDS-DMA, four stages,
// two tiles of lookahead) and read by the four waves.  The workgroup's key
// range is that of its last wave; the earlier waves see their extra tiles
// fully masked (about 1% of the products at 8192 positions).  One head per
// workgroup lets the four waves share the head's weights: the W_UK rows
// through the L1 cache, W_UV staged once in LDS for the epilogue.
#pragma once

#include <type_traits>

#include "prefill_bf16.h"
#include "solo_core.h"

namespace mla {

constexpr int kSoloWaves = 4;
constexpr int kSoloStages = 4;
constexpr int kSoloWaveRows = 32;                     // query positions per wave
constexpr int kSoloRows = kSoloWaveRows * kSoloWaves;  // per workgroup (one head)
constexpr int kSoloSpareBytes = 32768;  // LDS after the stages (the epilogue's gate rows)
constexpr int kSoloScoreLookahead = 2;
constexpr int kSoloValueLookahead = 2;

// q_abs^T blocks [blk0, blk1) of 32 latent dims from W_UK^T[h] held in LDS
// ([R, DQ] rows of DQ * 2 bytes, 16-byte chunk L of row j at L ^ (j & (DQ/8 - 1))),
// scaled by qscale: qT[kk] is the score B operand for k-block kk (lane column
// l % 32, latent dims 16 kk + 8 (l / 32) + 0..7).  qb[k] is the B operand q^T
// for d = 16 k + 8 (l / 32) + 0..7.  The A operand row rho of a block loads
// latent dim perm(rho) (bits 2 and 3 swapped) so that C registers 0-7 / 8-15
// of a lane are exactly the 8 consecutive dims of k-blocks 2 blk / 2 blk + 1.
// Two blocks run as interleaved chains, their operand reads two products
// ahead.
template <int DQ, int R>
__device__ __forceinline__ void absorb_lds(const MLA_LDS char* wk, const bf16x8 (&qb)[DQ / 16], float qscale,
                                           int lane, int blk0, int blk1, bf16x8 (&qT)[R / 16]) {
  constexpr int NKS = DQ / 16;
  static_assert(DQ / 8 <= 16, "chunk swizzle covers a row");
  const int l32 = lane & 31, hh = lane >> 5;
  const int prow = (l32 & 0x13) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
  const int xw = prow & (DQ / 8 - 1);
  const MLA_LDS char* base = wk + prow * (DQ * 2);
#pragma unroll
  for (int bp = blk0; bp < blk1; bp += 2) {
    // products p = 2 k + u of blocks bp + u
    auto operand = [&](int p) {
      return lds_read_b128(base + 32 * (bp + (p & 1)) * (DQ * 2) + (((2 * (p >> 1) + hh) ^ xw) << 4));
    };
    bf16x8 ar[3];
    ar[0] = operand(0);
    ar[1] = operand(1);
    f32x16 acc[2];
#pragma unroll
    for (int p = 0; p < 2 * NKS; ++p) {
      if (p + 2 < 2 * NKS) ar[(p + 2) % 3] = operand(p + 2);
      if (p < 2) mfma32v_first(acc[p & 1], ar[p % 3], qb[0]);
      else mfma32v(acc[p & 1], ar[p % 3], qb[p >> 1]);
    }
    settle_v(acc[0]);
    settle_v(acc[1]);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      qT[2 * (bp + u)] = pack8(acc[u], 0, qscale);
      qT[2 * (bp + u) + 1] = pack8(acc[u], 8, qscale);
      // materialise the packed operands here: left to itself the compiler
      // sinks the scale-and-pack to the first use and keeps the fp32 values
      asm volatile("" : "+v"(qT[2 * (bp + u)]), "+v"(qT[2 * (bp + u) + 1]));
    }
  }
}

template <int DQ, int DV, int R, bool PAGED = false, bool VARLEN = false>
__global__ void __launch_bounds__(64 * kSoloWaves)
__attribute__((amdgpu_waves_per_eu(1, 1)))
mla_prefill_solo_kernel(PrefillArgs a) {
  using LT = LatentTile<R>;
  using SA = SoloAttn<R>;
  constexpr int NS = kSoloStages;
  constexpr int NW = kSoloWaves;
  constexpr int CPW = copies_per_wave<R>(NW);
  constexpr int NKK = SA::NKK, NLB = SA::NLB;
  // A key tile is KH latent tiles of 32 rows in consecutive halves of one
  // stage: 64 keys at r = 256, 32 at r = 512, so that every tile carries 32
  // score and 32 value products per wave whatever r is (the per-tile waits,
  // barrier and softmax bookkeeping then weigh the same against them).
  constexpr int KH = R <= 256 ? 2 : 1;
  constexpr int KT = 32 * KH;             // keys per tile
  constexpr int STB = KH * LT::BYTES;     // stage bytes
  constexpr int CPT = KH * CPW;           // copies per wave per tile
  constexpr int NG = KH * NKK;            // score products per tile
  constexpr int NV = 2 * KH * NLB;        // value products per tile
  static_assert(NG == 32 && NV == 32 && CPT <= 8, "tile schedule");
  // At r = 256 (registers to spare) the score chains start from -m_run
  // instead of zero, so the scores arrive relative to the running maximum
  // and the exponentials need no subtraction; at r = 512 the scores are
  // absolute and the exponentials subtract m_run.
  constexpr bool PRESHIFT = KH == 2;
  // products of lookahead for the LDS operand reads (score / value)
  constexpr int SPF = kSoloScoreLookahead, VPF = kSoloValueLookahead;
  static_assert(LT::COPIES % NW == 0, "copy split");
  static_assert(DQ % 16 == 0 && DV % 32 == 0, "shape");
  static_assert(NS >= 3 && NS <= 5 && CPT * (NS - 2) < 64, "stages and vmcnt range");
  __shared__ __attribute__((aligned(1024))) char smem_raw[NS * STB + kSoloSpareBytes];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;

  // ---- work item (128 positions of one head), heaviest query blocks first
  int x = blockIdx.x;
  if constexpr (!VARLEN) {
    if (a.queue) {
      // Items go out in the order workgroups start, so the XCDs that run at
      // a higher clock take more of them (the clock differs by XCD under
      // this load, and a fixed share per XCD waits for the slowest).  The
      // item is passed on through the first LDS word, which every wave has
      // read before the second barrier lets any copy into the stages start.
      if (threadIdx.x == 0) *(MLA_LDS unsigned*)smem = atomicAdd(a.queue, 1u);
      __syncthreads();
      const unsigned item = __builtin_amdgcn_readfirstlane(*(const MLA_LDS unsigned*)smem);
      __syncthreads();
      x = item < gridDim.x ? (int)item : x;  // a counter not cleared cannot send work out of range
    }
  }
  int tb, b, hg;
  if constexpr (VARLEN) {
    hg = x % a.nhg;
    const int i = x / a.nhg;
    if (i >= __builtin_amdgcn_readfirstlane(*a.nblocks)) return;  // the whole workgroup
    const int2 e = a.blocks[i];
    b = __builtin_amdgcn_readfirstlane(e.x);
    tb = __builtin_amdgcn_readfirstlane(e.y);
  } else if (a.xcd_remap && !a.queue) {
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
  const int l32 = lane & 31, hh = lane >> 5;
  const int h = hg;  // one head per workgroup (hg < H)
  constexpr bool hvalid = true;
  const int hc = h;
  const int H = a.H;
  int T = a.T, S = a.S;
  size_t qr0 = (size_t)b * a.T;  // packed row of query 0 of sequence b
  if constexpr (VARLEN) {
    const int4 sq = a.seq[b];
    qr0 = (size_t)__builtin_amdgcn_readfirstlane(sq.x);
    T = __builtin_amdgcn_readfirstlane(sq.y);
    S = __builtin_amdgcn_readfirstlane(sq.z);
  }
  const int t0 = tb * kSoloRows;           // first query of the workgroup
  const int tw = t0 + kSoloWaveRows * w;   // first query of this wave
  const int t = tw + l32;  // this lane's query column
  const bool tvalid = t < T;
  const int P = S - T;  // query t sits at position P + t
  const int kend = P + min(t0 + kSoloRows, T);  // keys [0, kend) reach a query of the workgroup
  const int ntiles = (kend + KT - 1) / KT;

  TileCopier<R, NW, 1> copier;
  copier.init(w, lane);

  // copies of the 32-row half hf of key tile j into its stage; halves past
  // the keys the workgroup needs are copied as zero rows
  auto prepare_half = [&](int j, int hf, bool with_lane_base = true) {
    const int jj = KH * j + hf;
    return prepare_key_tile<PAGED>(copier, a, b, S, jj, smem + (j % NS) * STB + hf * LT::BYTES, 32 * jj < kend,
                                   with_lane_base);
  };
  auto issue_tile = [&](int j) {
#pragma unroll
    for (int hf = 0; hf < KH; ++hf) copier.template issue_range<0, CPW>(prepare_half(j, hf));
  };

  // ---- absorb.  W_UK^T[h] ([R, DQ], 128 KiB at full width) is staged in the
  // LDS stages by the four waves together (1 KiB LDS-DMA copies) in four
  // chunks of R/4 rows, one per stage, and each wave's 32 query rows in the
  // region after the stages.  Each wave forms its q_abs^T chunk by chunk as
  // the chunks land; stage c then takes latent tile c (tiles 0 .. NS-2).
  // Every load here is an LDS-DMA copy with an explicit wait count (a
  // compiler-visible load would get a vmcnt(0) that also waits for the
  // copies issued after it).
  constexpr int WKB = R * DQ * 2;                 // W_UK^T bytes
  constexpr int CPRW = DQ / 8;                    // 16-byte chunks per W_UK^T / q row
  constexpr int WCC = WKB / NS / 1024 / NW;       // copies per wave per chunk
  constexpr int QCW = 32 * DQ * 2 / 1024;         // q copies per wave
  constexpr int NKS = DQ / 16;
  constexpr int WCB = WKB / NS;                    // W_UK^T chunk bytes (chunk c sits in stage c)
  static_assert(WKB % (NS * NW * 1024) == 0 && WCB <= STB && NS == 4 && 64 % CPRW == 0 && CPRW <= 16,
                "W_UK^T chunks fit the stages");
  static_assert(NW * QCW * 1024 <= kSoloSpareBytes && NS * WCC + QCW < 64, "q staging");
  MLA_LDS char* qbuf = smem + NS * STB + w * (QCW * 1024);
  {
    unsigned ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    const unsigned rsub = ln / CPRW, cl = ln % CPRW;
    // q rows tw + r of head h (rows past T repeat row T - 1): row r at
    // r DQ 2 bytes, chunk L at L ^ (r & (CPRW - 1))
    const u32x4 qrs = make_rsrc(a.q + qr0 * (size_t)H * DQ + (size_t)hc * DQ, (unsigned)((size_t)T * H * DQ * 2));
#pragma unroll
    for (int i = 0; i < QCW; ++i) {
      const unsigned r = (64 / CPRW) * i + rsub;
      const unsigned row = (unsigned)min(tw + (int)r, T - 1);
      buf2lds16(qrs, (row * (unsigned)(H * DQ) + ((cl ^ (r & (CPRW - 1))) * 8)) * 2, qbuf + i * 1024);
    }
    const u32x4 krs = make_rsrc(a.wukT + (size_t)hc * R * DQ, (unsigned)WKB);
#pragma unroll
    for (int c = 0; c < NS * WCC; ++c) {
      const int i = c * NW + w;  // copy i: rows (64 / CPRW) i .. (chunk c / WCC)
      const unsigned row = (64 / CPRW) * i + rsub;
      const int ch = i / (NW * WCC);
      buf2lds16(krs, (row * DQ + ((cl ^ (row & (CPRW - 1))) * 8)) * 2,
                smem + ch * STB + (i - ch * NW * WCC) * 1024);
    }
  }
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
  bf16x8 qT[NKK];
  bf16x8 qb[NKS];
  constexpr int BPC = NLB / NS;  // 32-row latent blocks per chunk
  // chunk 0 (and the q rows, copied first)
  wait_vmcnt<(NS - 1) * WCC>();
  wg_barrier();
#pragma unroll
  for (int k = 0; k < NKS; ++k)
    qb[k] = lds_read_b128(qbuf + l32 * (DQ * 2) + (((2 * k + hh) ^ (l32 & (CPRW - 1))) << 4));
  // rows of chunk c sit in stage c: the base of chunk c's rows as if the
  // chunks were contiguous
  auto wk_base = [&](int c) { return smem + c * (STB - WCB); };
  absorb_lds<DQ, R>(wk_base(0), qb, a.qscale, lane, 0, BPC, qT);
  // chunk c + 1 has landed once at most the younger chunks (NS - 2 - c of
  // them) and tiles 0 .. c - 1 (two chunks' worth of copies each) are
  // outstanding; the barrier also frees stage c for tile c.  Tiles past the
  // last are copied as zero rows (no branches; every step below then has
  // exactly NS - 3 younger tiles in flight).
  wait_vmcnt<(NS - 2) * WCC>();
  wg_barrier();
  issue_tile(0);
  absorb_lds<DQ, R>(wk_base(1), qb, a.qscale, lane, BPC, 2 * BPC, qT);
  wait_vmcnt<(NS - 3) * WCC + CPT>();
  wg_barrier();
  issue_tile(1);
  absorb_lds<DQ, R>(wk_base(2), qb, a.qscale, lane, 2 * BPC, 3 * BPC, qT);
  wait_vmcnt<2 * CPT>();
  wg_barrier();
  issue_tile(2);
  absorb_lds<DQ, R>(wk_base(3), qb, a.qscale, lane, 3 * BPC, 4 * BPC, qT);
  float m_run, l_run = 0.0f;

  // causal mask of the 32 keys from s0 (also hides keys past S); key of
  // register r is s0 + 8 (r / 4) + 4 (l / 32) + r % 4
  auto mask = [&](f32x16& s, int s0) __attribute__((always_inline)) {
    if (s0 + 31 > P + tw) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (s0 + 8 * (r >> 2) + 4 * hh + (r & 3) > P + t) s[r] = -INFINITY;
    }
  };
  // column maximum of 32 keys and v over this lane's 16 keys; the other 16
  // sit in lane l ^ 32 (xhalf_max)
  auto lane_max = [&](const f32x16& s, float v) {
    const float m0 = max3_nn(s[0], s[1], s[2]), m1 = max3_nn(s[3], s[4], s[5]);
    const float m2 = max3_nn(s[6], s[7], s[8]), m3 = max3_nn(s[9], s[10], s[11]);
    const float m4 = max3_nn(s[12], s[13], s[14]);
    return max3_nn(max3_nn(m0, m1, m2), max3_nn(m3, m4, s[15]), v);
  };
  auto tile_at = [&](int j) { return smem + (j % NS) * STB; };
  // score operand g of a tile: k-block g % NKK of its half g / NKK
  auto score_op = [&](const MLA_LDS char* tile, int g) {
    return sa.score_operand(tile + (g / NKK) * LT::BYTES, g % NKK);
  };


  // ---- tile 0: scores only (each step below starts with its tile's softmax)
  wait_vmcnt<(NS - 2) * CPT>();  // tile 0 landed (tiles 1 .. NS-2 may be in flight)
  wg_barrier();
  f32x16 sc[KH];
  {
    bf16x8 ao[3];
    ao[0] = score_op(smem, 0);
    ao[1] = score_op(smem, 1);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g + 2 < NG) ao[(g + 2) % 3] = score_op(smem, g + 2);
      __builtin_amdgcn_sched_barrier(0);
      if (g % NKK == 0) mfma32v_first(sc[g / NKK], ao[g % 3], qT[0]);
      else mfma32v(sc[g / NKK], ao[g % 3], qT[g % NKK]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int hf = 0; hf < KH; ++hf) {
    settle_v(sc[hf]);
    mask(sc[hf], 32 * hf);
    mx = lane_max(sc[hf], mx);
  }
  mx = xhalf_max(mx);
  m_run = mx;
  // -m_run in every accumulator slot (the chains' start with PRESHIFT)
  f32x16 negm;
  auto set_negm = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) negm[i] = -m_run;
    asm volatile("" : "+v"(negm));
    operand_gap();
  };
  if constexpr (PRESHIFT) {
#pragma unroll
    for (int hf = 0; hf < KH; ++hf)
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[hf][i] -= m_run;
    mx = 0.0f;
    set_negm();
  }

  // The reference max moves only when a score exceeds it by more than 8 (so
  // P <= 2^8): the O^T rescale is rare.  Every lane of a column pair holds
  // the same maxima, so both halves take the same decision.
  auto maybe_rescale = [&](f32x16 (&sc)[KH]) __attribute__((always_inline)) {
    if constexpr (PRESHIFT) {
      // mx and the scores of tile it are relative to m_run
      const bool need = mx > 8.0f;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float d = need ? mx : 0.0f;
        const float alpha = fast_exp2(-d);
        l_run *= alpha;
        wait_states_24();  // the last value products have written O^T
#pragma unroll
        for (int u = 0; u < NLB; ++u) scale_acc(oT[u], alpha);
        wait_states_24();  // the rescaled O^T feeds the next value products
        m_run += d;
#pragma unroll
        for (int hf = 0; hf < KH; ++hf)
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[hf][i] -= d;
        set_negm();
      }
    } else {
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
    }
  };
  // p = 2^(s - m_run) for a score s of tile it
  auto expo = [&](float s_) __attribute__((always_inline)) {
    if constexpr (PRESHIFT) return fast_exp2(s_);
    else return fast_exp2(s_ - m_run);
  };

  // This wave's lane offsets of its copies of a tile, formed once here
  // instead of at every tile (the tile's descriptor changes, they do not).
  unsigned coff[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) coff[c] = copier.offset_of(w + NW * c);

  // One key tile `it`: on entry sc holds the masked scores of tile it and mx
  // their column maxima; on exit, those of tile it+1 (garbage after the last
  // tile, never used).  Score product g (k-block g % NKK of half g / NKK) and
  // value product n (latent block n % NLB, key block n / NLB) number the
  // tile's 32 + 32 products.  masked (a BoolTag) says whether tile it+1
  // needs the causal mask; the steps before the diagonal run without it.
  auto step_next = [&](int it, auto masked, f32x16 (&sc)[KH], f32x16 (&sn)[KH]) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    const MLA_LDS char* tile = tile_at(it);
    const MLA_LDS char* tnext = tile_at(it + 1);
    // tile it+1 landed; tiles it+2 .. it+NS-2 may still be in flight
    wait_vmcnt<(NS - 3) * CPT>();
    wg_barrier();  // tile it+1 visible; every wave is done with tile it-1
    // the first score operands of tile it+1 go out before anything else, and
    // the first value operands of tile it (resident since the last step)
    // right after: their LDS latency runs under the bookkeeping below
    bf16x8 ao[SPF + 1], av[VPF + 1];
#pragma unroll
    for (int u = 0; u < SPF; ++u) ao[u] = score_op(tnext, u);
#pragma unroll
    for (int u = 0; u < VPF; ++u) av[u] = sa.value_operand(tile, u);
    // tile it+NS-1 goes into the stage tile it-1 has left; its copies are
    // spread over phase B, one after every fourth value product (sent all at
    // once they stall the wave for several hundred cycles).  Past the last
    // tile they are issued anyway, with an empty range that writes zeros
    // into that free stage: a branch around each copy costs more than it.
    typename TileCopier<R, NW, 1>::Pending pend[KH];
#pragma unroll
    for (int hf = 0; hf < KH; ++hf) pend[hf] = prepare_half(it + NS - 1, hf, false);
    maybe_rescale(sc);

    // phase A: score products 0 .. NG/2-1 of tile it+1 (operands read SPF
    // products ahead) under the exponentials of half 0 of tile it; those of
    // half 1 (r = 256) run under the first phase-B slots
#pragma unroll
    for (int g = 0; g < NG / 2; ++g) {
      ao[(g + SPF) % (SPF + 1)] = score_op(tnext, g + SPF);
      __builtin_amdgcn_sched_barrier(0);
      if (g % NKK == 0) {
        if constexpr (PRESHIFT) mfma32v_init(sn[g / NKK], ao[g % (SPF + 1)], qT[0], negm);
        else mfma32v_first(sn[g / NKK], ao[g % (SPF + 1)], qT[0]);
      } else {
        mfma32v(sn[g / NKK], ao[g % (SPF + 1)], qT[g % NKK]);
      }
      sc[0][g] = expo(sc[0][g]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // P is packed by VALU instructions: each quarter is materialised where it
    // is formed (the compiler would otherwise sink it towards its products,
    // past the gap) and read by a product at least two wait states later
    bf16x8 pB[2 * KH];
    pB[0] = pack8(sc[0], 0, 1.0f);
    asm volatile("" : "+v"(pB[0]));
    operand_gap();
    // phase B: value products of tile it in key-block-major order, so the
    // first NLB use only the first quarter of P; the first NG/2 are each
    // followed by one of the remaining score products of tile it+1
    float m_half = -INFINITY;
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      // the score operand of slot n + SPF goes out before the value operand
      // of slot n + VPF: the wait for a slot's value operand then covers its
      // score operand too (one s_waitcnt per slot)
      if (n < NG / 2 && NG / 2 + n + SPF < NG) ao[(NG / 2 + n + SPF) % (SPF + 1)] = score_op(tnext, NG / 2 + n + SPF);
      __builtin_amdgcn_sched_barrier(0);
      if (n + VPF < NV) av[(n + VPF) % (VPF + 1)] = sa.value_operand(tile, n + VPF);
      __builtin_amdgcn_sched_barrier(0);
      mfma32a(oT[n % NLB], av[n % (VPF + 1)], pB[n / NLB]);
      __builtin_amdgcn_sched_barrier(0);
      if ((n & 3) == 1 && (n >> 2) < CPT) {
        const int c = (n >> 2) % CPW;
        buf2lds16(pend[(n >> 2) / CPW].rs, coff[c], pend[(n >> 2) / CPW].stage + (w + NW * c) * 1024);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (n < NG / 2) {
        const int g = NG / 2 + n;
        if (g % NKK == 0) {
          if constexpr (PRESHIFT) mfma32v_init(sn[g / NKK], ao[g % (SPF + 1)], qT[0], negm);
          else mfma32v_first(sn[g / NKK], ao[g % (SPF + 1)], qT[0]);
        } else {
          mfma32v(sn[g / NKK], ao[g % (SPF + 1)], qT[g % NKK]);
        }
        if constexpr (KH == 2) sc[1][n] = expo(sc[1][n]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // the rest of the softmax of tile it, and the mask and column maxima
      // of tile it+1 once its scores are complete, each under one product
      if (n == 0) {
        pB[1] = pack8(sc[0], 8, 1.0f);
        asm volatile("" : "+v"(pB[1]));
        __builtin_amdgcn_sched_barrier(0);
      }
      if (n == 1) {
        l_run = sum8_bf16(pB[1], sum8_bf16(pB[0], l_run));
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (KH == 2) {
        if (n == NG / 4) {  // exponentials 0 .. 7 of half 1 are done
          pB[2] = pack8(sc[1], 0, 1.0f);
          asm volatile("" : "+v"(pB[2]));
          __builtin_amdgcn_sched_barrier(0);
        }
        if (n == NG / 2) {
          pB[3] = pack8(sc[1], 8, 1.0f);
          asm volatile("" : "+v"(pB[3]));
          __builtin_amdgcn_sched_barrier(0);
        }
        if (n == NG / 2 + 1) {
          l_run = sum8_bf16(pB[3], sum8_bf16(pB[2], l_run));
          __builtin_amdgcn_sched_barrier(0);
        }
        // half 0 of tile it+1 is complete after phase A
        if (n == 2) {
          settle_v(sn[0]);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (n == 3) {
          if constexpr (MASKED) mask(sn[0], (it + 1) * KT);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (n == 4) {
          m_half = lane_max(sn[0], -INFINITY);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // the last half of tile it+1 is complete after phase-B slot NG/2 - 1
      if (n == NG / 2 + KH) {
        settle_v(sn[KH - 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (n == NG / 2 + KH + 1) {
        if constexpr (MASKED) mask(sn[KH - 1], (it + 1) * KT + 32 * (KH - 1));
        __builtin_amdgcn_sched_barrier(0);
      }
      if (n == NG / 2 + KH + 2) {
        mx = xhalf_max(lane_max(sn[KH - 1], m_half));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };


  // Every tile runs the same step, the last one included: its look-ahead
  // score products read a stage no copy is writing (stale bytes) and are
  // discarded, about half a tile of extra products per workgroup.  A peeled
  // last step after the loop would be cheaper in products, but the extra live
  // ranges push the architectural registers over 256 and the allocator then
  // evicts O^T from its registers; a branch inside the loop whose arms both
  // update O^T does the same at its join.
  // Tiles 0 .. nfull-1 hold no key past this wave's first query, so the
  // steps that form their scores need no mask (wave-uniform; every wave
  // still runs ntiles steps and meets the same barriers).
  const int nfull = (P + tw + 1) / KT;
  const int nfree = min(max(nfull - 1, 0), ntiles);
  // The scores alternate between two register sets, two steps per
  // iteration (a copy of the next tile's scores at every step would cost as
  // many moves); an odd last mask-free step runs with the masked ones (the
  // mask changes nothing on a tile wholly before the wave's queries).
  f32x16 sc2[KH];
  int it = 0;
  for (; it + 1 < nfree; it += 2) {
    step_next(it, BoolTag<false>{}, sc, sc2);
    step_next(it + 1, BoolTag<false>{}, sc2, sc);
  }
  for (; it < ntiles; ++it) {
    step_next(it, BoolTag<true>{}, sc, sc2);
#pragma unroll
    for (int hf = 0; hf < KH; ++hf) sc[hf] = sc2[hf];
  }

  // ---- epilogue: o^T = W_UV[h] (O^T / l), gate, store
  // W_UV[h] ([DV, R], 64 KiB to 128 KiB) is staged whole in the stages by the
  // four waves together (row v at v R 2 bytes, chunk L at L ^ (v & 15)), and
  // each wave's 32 gate rows (DV logits each) in the region after them (row
  // r at r DV 2 bytes, chunk L at L ^ (r & (DV/8 - 1))): every load of the epilogue
  // is an LDS-DMA copy, waited for with explicit counts.  The copies go out
  // first; O^T is normalised and packed under them.
  constexpr int NVB = DV / 32;
  constexpr int CPR = R / 8;                  // 16-byte chunks per W_UV row
  constexpr int RPC = 64 / CPR;               // W_UV rows per 1 KiB copy
  constexpr int CPV = 32 / RPC / NW;          // copies per wave per v-block
  constexpr int GCR = DV / 8;                 // 16-byte chunks per gate row
  constexpr int GCW = 32 * DV * 2 / 1024;     // gate copies per wave
  static_assert(DV * R * 2 <= NS * STB && CPV >= 1 && CPV * NVB + GCW < 64, "W_UV staging");
  static_assert(64 % GCR == 0 && GCR <= 16 && NW * GCW * 1024 <= kSoloSpareBytes, "gate staging");
  MLA_LDS char* gbuf = smem + NS * STB + w * (GCW * 1024);
  wait_vmcnt<0>();  // the zero-row copies of the tiles past the last write the stages
  wg_barrier();     // every wave is done with the key tiles
  {
    unsigned ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    // gate rows tw + r of head h (rows past T repeat row T - 1)
    const u32x4 grs = make_rsrc(a.gate + qr0 * (size_t)H * DV + (size_t)hc * DV, (unsigned)((size_t)T * H * DV * 2));
    const unsigned gsub = ln / GCR, gcl = ln % GCR;
#pragma unroll
    for (int i = 0; i < GCW; ++i) {
      const unsigned r = (64 / GCR) * i + gsub;
      const unsigned row = (unsigned)min(tw + (int)r, T - 1);
      buf2lds16(grs, (row * (unsigned)(H * DV) + ((gcl ^ (r & (GCR - 1))) * 8)) * 2, gbuf + i * 1024);
    }
    const u32x4 wrs = make_rsrc(a.wuv + (size_t)hc * DV * R, (unsigned)(DV * R * 2));
    const unsigned rsub = ln / CPR, cl = ln % CPR;
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
      for (int c = 0; c < CPV; ++c) {
        const int i = (vb * CPV + c) * NW + w;  // copy index: rows RPC i ..
        const unsigned row = RPC * i + rsub;
        buf2lds16(wrs, (row * R + ((cl ^ (row & 15)) * 8)) * 2, smem + i * 1024);
      }
  }
  wait_states_24();  // the last value products have written O^T
#pragma unroll
  for (int u = 0; u < NLB; ++u) pin_a(oT[u]);
  const float l_tot = xhalf_sum(l_run);
  const float inv_l = 1.0f / l_tot;
  if (a.lse && hh == 0 && tvalid && hvalid)
    a.lse[((size_t)b * H + h) * T + t] = (m_run + __builtin_log2f(l_tot)) * 0.69314718055994531f;
  const bool store = tvalid && hvalid;
  const size_t orow = (qr0 + (tvalid ? t : T - 1)) * (size_t)H * DV + (size_t)hc * DV;
  // O^T is packed unnormalised (bf16 keeps the same relative precision) and
  // 1/l is applied to the products instead: 16 values per v-block and lane
  // rather than 16 per latent block
  bf16x8 ob[2 * NLB];
#pragma unroll
  for (int u = 0; u < NLB; ++u) {
    ob[2 * u] = pack8(oT[u], 0, 1.0f);
    ob[2 * u + 1] = pack8(oT[u], 8, 1.0f);
    // packed here, not sunk into the products below, where the fp32 values
    // would hold the registers the operand reads run ahead in
    asm volatile("" : "+v"(ob[2 * u]), "+v"(ob[2 * u + 1]));
  }
  // this lane's gate logits v = 32 vb + 8 c + 4 (l / 32) + 0..3 of row l32
  const MLA_LDS char* grow = gbuf + l32 * (DV * 2) + 8 * hh;
  const MLA_LDS char* wrow = smem + l32 * (R * 2) + 8 * hh;  // + 32 vb R 2
  // All of W_UV and the gate rows have landed by now (the packing above
  // runs under the copies), so one wait and one barrier cover them, and the
  // v-blocks run as NVB independent chains over the shared O^T operands:
  // the operand reads run ahead of the products and the products issue
  // back to back.
  wait_vmcnt<0>();
  wg_barrier();  // W_UV and the gate rows copied by every wave
  f32x16 acc[NVB];
  // k-block kb = latent 16 kb + 8 c + 4 (l / 32) + e for slot 4 c + e; the
  // operands of k-block kb + 1 are read while the products of kb issue.
  // The products are compiler builtins (their register hazards stay the
  // compiler's), fenced by scheduling barriers so that the reads stay a
  // k-block ahead instead of being sunk to each product.
  bf16x8 wop[2][NVB];
  auto read_w = [&](int kb, bf16x8 (&o)[NVB]) {
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      const MLA_LDS char* rb = wrow + vb * 32 * (R * 2);
      const bf16x4 lo = *(const MLA_LDS bf16x4*)(rb + (((2 * kb) ^ (l32 & 15)) << 4));
      const bf16x4 hi = *(const MLA_LDS bf16x4*)(rb + (((2 * kb + 1) ^ (l32 & 15)) << 4));
      o[vb] = cat4(lo, hi);
    }
  };
  read_w(0, wop[0]);
#pragma unroll
  for (int kb = 0; kb < 2 * NLB; ++kb) {
    if (kb + 1 < 2 * NLB) read_w(kb + 1, wop[(kb + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb)
      acc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wop[kb & 1][vb], ob[kb], kb == 0 ? f32x16{} : acc[vb], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (store) {
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bf16x4 ov;
        const bf16x4 gl = *(const MLA_LDS bf16x4*)(grow + (((4 * vb + c) ^ (l32 & (GCR - 1))) << 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (bf16)(acc[vb][4 * c + e] * (inv_l * sigmoidf_((float)gl[e])));
        *(bf16x4*)(a.out + orow + 32 * vb + 8 * c + 4 * hh) = ov;
      }
  }
}

}  // namespace mla
