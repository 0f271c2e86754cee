// bf16 decode kernels for the absorbed Gated MLA layer on gfx950: one new
// query per sequence attends to its whole cached latent (the cache holds only
// c, page "Gated MLA（矩阵吸收版）", section 低秩压缩 and the KV-cache table of
// section 形状与参数对比).  The pages stop short of a decode path; this one
// evaluates the same definition as prefill for the last position.
//
//  mla_decode_absorb    q_abs[i, h, :] = scale*log2e * q[i, h, :] W_UK[h], read
//                       straight from W_UK [H, DQ, R] (no transposed copy)
//  mla_decode_split     the packed cache rows are cut into G equal ranges, one
//                       per workgroup; each range is streamed from HBM into
//                       LDS once and scored against all H heads (heads are the
//                       MFMA columns, 16 per wave, up to 8 waves).  Every
//                       sequence piece in a range leaves an unnormalised
//                       partial (m, l in fp32, O[r] in bf16).
//  mla_decode_merge     per (head, 16 sequences): log-sum-exp merge of the
//                       partials, then o = o_lat W_UV[h]^T on MFMA, the
//                       sigmoid gate and the store.
//
// Range k covers cache rows [floor(k*N/G), floor((k+1)*N/G)); the partial of
// sequence i from range k is stored in slot k + i, which is unique because
// the sequences met by consecutive ranges are consecutive.
#pragma once

#include <type_traits>

#include "attn_core.h"

namespace mla {

// ----------------------------------------------------------------- W_UK^T
template <typename T>
__global__ void __launch_bounds__(256) mla_wuk_transpose(const T* __restrict__ w, T* __restrict__ wt,
                                                         int DQ, int R, unsigned* queue) {
  // one 32 (d) x 32 (j) tile per workgroup (head blockIdx.z): read rows of W_UK[h], write rows of W_UK^T[h]
  __shared__ T tile[32][33];
  // the prefill that follows on the stream takes its work items from *queue
  if (queue && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) *queue = 0u;
  const int h = blockIdx.z;
  const int j0 = blockIdx.x * 32, d0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  const T* src = w + (size_t)h * DQ * R;
  T* dst = wt + (size_t)h * R * DQ;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int d = d0 + ty + 8 * k, j = j0 + tx;
    if (d < DQ && j < R) tile[ty + 8 * k][tx] = src[(size_t)d * R + j];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int j = j0 + ty + 8 * k, d = d0 + tx;
    if (d < DQ && j < R) dst[(size_t)j * DQ + d] = tile[tx][ty + 8 * k];
  }
}

// One workgroup (256 threads): clamps the lengths to [1, max_rows] and writes them, the
// exclusive prefix sums of the tile counts (cu_t[B] = NT) and the number of
// ranges cu_t[B + 1] = min(G, NT), so that no range is empty (the merge walks
// every range between a sequence's first and last).  The lengths come from
// seq_lens, or (cu != nullptr, packed cache) from the row prefix sums
// cu[i + 1] - cu[i].  The sums run in 64 bits and are capped at 2^30 tiles,
// which only lengths that break the callers' preconditions reach: the prefix
// sums stay monotone whatever the lengths, and sequences past the cap get no
// tiles.
//
// With rt != nullptr the G ranges are cut by cost instead: a tile costs 1 and
// the start of a sequence switch_tiles more (a workgroup that reaches a new
// sequence stores a partial and loads that sequence's query), so ranges that
// cross many sequence starts take fewer tiles.  Range k covers tiles
// [rt[k], rt[k + 1]) (rt[G] = NT; a range may be empty), and krange[2i],
// krange[2i + 1] are the first and last range holding tiles of sequence i.
// When B + G + 2 <= kPrepareLds the binary searches read LDS copies of cu_t
// and rt instead of the global arrays just written (a few hundred cycles per
// step less).
constexpr int kPrepareLds = 2048;

struct PrepareArgs {
  const int* seq_lens;  // [B] (paged), or
  const int* cu;        // [B + 1] row prefix sums (packed)
  int B, max_rows, G;
  int* lens;            // [B]
  int* cu_t;            // [B + 2]
  int* rt;              // [G + 1] or null
  int* krange;          // [B, 2] (with rt)
  int switch_tiles;
};

__device__ __forceinline__ void decode_prepare(const PrepareArgs& pa) {
  const int* __restrict__ seq_lens = pa.seq_lens;
  const int* __restrict__ cu = pa.cu;
  const int B = pa.B, max_rows = pa.max_rows, G = pa.G;
  int* __restrict__ lens = pa.lens;
  int* __restrict__ cu_t = pa.cu_t;
  int* __restrict__ rt = pa.rt;
  int* __restrict__ krange = pa.krange;
  const int switch_tiles = pa.switch_tiles;
  constexpr long long kCap = 1LL << 30;
  __shared__ long long wsum[4];
  __shared__ int s_cut[kPrepareLds];  // cu_t[0..B], then rt[0..G]
  const bool in_lds = B + G + 2 <= kPrepareLds;  // uniform
  int* s_rt = s_cut + (in_lds ? B + 1 : 0);
  auto cut = [&](int i) { return in_lds ? s_cut[i] : cu_t[i]; };
  auto rts = [&](int k) { return in_lds ? s_rt[k] : rt[k]; };
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  long long carry = 0;
  if (tid == 0) {
    cu_t[0] = 0;
    if (in_lds) s_cut[0] = 0;
  }
  for (int base = 0; base < B; base += 256) {
    const int i = base + tid;
    long long tiles = 0;
    if (i < B) {
      long long len = cu ? (long long)cu[i + 1] - cu[i] : (long long)seq_lens[i];
      len = len < 1 ? 1 : (len > max_rows ? max_rows : len);
      tiles = (len + 31) / 32;
      lens[i] = (int)len;
    }
    long long incl = tiles;  // inclusive scan inside the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const long long v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    long long before = carry;
    for (int u = 0; u < w; ++u) before += wsum[u];
    if (i < B) {
      const int v = (int)min(before + incl, kCap);
      cu_t[i + 1] = v;
      if (in_lds) s_cut[i + 1] = v;
    }
    carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  const long long NT = min(carry, kCap);
  if (tid == 0) cu_t[B + 1] = (int)min((long long)G, NT);
  if (!rt) return;
  __syncthreads();  // cu_t complete
  // cost of everything before sequence i: cu_t[i] + S i; range k < Ge starts
  // at cost floor(k C / Ge), C = NT + S B, inside sequence i: at its first
  // tile while in the sequence's start cost, else after (cost - S) of its
  // tiles.  Ge = min(G, C) keeps every range at least one cost unit wide, so
  // only ranges inside a start cost are empty (none lies within a
  // sequence's tiles); the ranges from Ge on are empty and past the end.
  const long long S = switch_tiles, C = NT + S * B;
  const long long Ge = min((long long)G, C);
  for (int k = tid; k <= G; k += 256) {
    int t = (int)NT;
    if (k < Ge) {
      const long long c = (long long)k * C / Ge;
      int l = 0, r = B - 1;  // the largest i with cu_t[i] + S i <= c
      while (l < r) {
        const int mid = (l + r + 1) >> 1;
        if ((long long)cut(mid) + S * mid <= c) l = mid; else r = mid - 1;
      }
      const long long cl = cut(l);
      const long long off = c - (cl + S * l);
      t = (int)(off < S ? cl : min(cl + (off - S), (long long)cut(l + 1)));
    }
    rt[k] = t;
    if (in_lds) s_rt[k] = t;
  }
  __syncthreads();  // rt complete
  for (int i = tid; i < B; i += 256) {
    // the range holding tile x: the largest k < G with rt[k] <= x
    auto range_at = [&](int x) {
      int l = 0, r = G - 1;
      while (l < r) {
        const int mid = (l + r + 1) >> 1;
        if (rts(mid) <= x) l = mid; else r = mid - 1;
      }
      return l;
    };
    krange[2 * i] = range_at(cut(i));
    krange[2 * i + 1] = range_at(cut(i + 1) - 1);
  }
}

__global__ void __launch_bounds__(256) mla_paged_prepare(PrepareArgs pa) { decode_prepare(pa); }

// ----------------------------------------------------------------- absorb
struct DecodeAbsorbArgs {
  const bf16* q;    // [B, H, DQ]
  const bf16* wuk;  // [H, DQ, R]
  bf16* qabs;       // [B, H, R]
  int B, H;
  float qscale;
  int with_prep;    // workgroup 0 runs decode_prepare(prep) instead
  PrepareArgs prep;
};

// Workgroup (head h, latent columns [J0, J0 + JC)), 4 waves; wave w owns the
// 16 latent columns J0 + 16w .. and walks the sequences 64 at a time (the
// queries of all 64 in flight together, the first 64 before the W_UK slice
// is staged): q_abs^T[j, i] = sum_d W_UK[h, d, j] q[i, h, d] on MFMA.  The
// W_UK slice [DQ x JC] is staged in LDS as stored (d-major); the A operand
// (row j, 8 consecutive d) comes from two transposing ds_read_b64_tr_b16
// reads.  Output rows are stored in the plain [B, H, R] layout, scaled by
// qscale.
template <int DQ, int R>
__global__ void __launch_bounds__(256) mla_decode_absorb(DecodeAbsorbArgs a) {
  constexpr int JC = R < 64 ? R : 64;    // latent columns per workgroup
  constexpr int DP = DQ < 32 ? 32 : DQ;  // staged rows, zero-padded to a whole k-step
  constexpr int NK = DP / 32;
  constexpr int LD = JC + 8;             // padded row (elements): spreads the tr16 rows over banks
  static_assert(R % JC == 0 && JC % 16 == 0 && DQ % 8 == 0, "absorb tiling");
  constexpr int IT = 4;                  // 16-sequence blocks in flight
  __shared__ __attribute__((aligned(16))) bf16 wt[DP][LD];
  // The range table's workgroup is block 0, so that its chain of dependent
  // steps starts with the first blocks rather than after the last.
  if (a.with_prep && blockIdx.x == 0) {
    decode_prepare(a.prep);
    return;
  }
  const int bx = blockIdx.x - a.with_prep;
  const int h = bx / (R / JC), J0 = (bx % (R / JC)) * JC;
  const bf16* __restrict__ src = a.wuk + (size_t)h * DQ * R + J0;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, kq = lane >> 4;
  bf16x8 bq[IT][NK];
  auto load_q = [&](int i00) {
#pragma unroll
    for (int t = 0; t < IT; ++t) {
      const int i = i00 + 16 * t + l16;
      const bf16* qrow = a.q + ((size_t)(i < a.B ? i : a.B - 1) * a.H + h) * DQ;
#pragma unroll
      for (int k = 0; k < NK; ++k)
        bq[t][k] = (32 * k + 8 * kq < DQ) ? *(const bf16x8*)(qrow + 32 * k + 8 * kq) : bf16x8{};
    }
  };
  load_q(0);
  for (int e = threadIdx.x; e < DP * JC / 8; e += 256) {
    const int d = e / (JC / 8), j8 = e % (JC / 8);
    const bf16x8 v = d < DQ ? *(const bf16x8*)(src + (size_t)d * R + 8 * j8) : bf16x8{};
    *(bf16x8*)&wt[d][8 * j8] = v;
  }
  __syncthreads();
  if (16 * w >= JC) return;
  const int e4 = l16 >> 2, q4 = l16 & 3;
  bf16x8 af[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const int d = 32 * k + 8 * kq + e4;
    af[k] = cat4(lds_read_tr16((const MLA_LDS char*)&wt[d][16 * w + 4 * q4]),
                 lds_read_tr16((const MLA_LDS char*)&wt[d + 4][16 * w + 4 * q4]));
  }
  for (int i00 = 0;;) {
#pragma unroll
    for (int t = 0; t < IT; ++t) {
      const int i = i00 + 16 * t + l16;
      f32x4 acc = f32x4{};
#pragma unroll
      for (int k = 0; k < NK; ++k) acc = mfma16(af[k], bq[t][k], acc);
      if (i < a.B) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(acc[e] * a.qscale);
        *(bf16x4*)(a.qabs + ((size_t)i * a.H + h) * R + J0 + 16 * w + 4 * kq) = v;
      }
    }
    i00 += 16 * IT;
    if (i00 >= a.B) break;
    load_q(i00);
  }
}

// ----------------------------------------------------------------- split
struct DecodeSplitArgs {
  const bf16* qabs;     // [B, H, R]
  const bf16* cache;    // [N, R]
  const int* cu;        // [B + 1]
  bf16* part_o;         // [(G + B), H, R]  unnormalised O, bf16
  float* part_ml;       // [(G + B), H, 2]
  int B, H, G;
  long long N;          // cache rows (total_len)
};

__device__ __forceinline__ long long range_start(long long k, long long N, long long G) {
  return k * N / G;
}

constexpr int kDecodeWaves = 8;
constexpr int kDecodeStages = 4;  // 3 tiles in flight cover HBM latency

template <int R>
__global__ void __launch_bounds__(64 * kDecodeWaves)
__attribute__((amdgpu_waves_per_eu(2, 2)))
mla_decode_split(DecodeSplitArgs a) {
  using LT = LatentTile<R>;
  constexpr int NS = kDecodeStages;
  constexpr int LPW = copies_per_wave<R>(kDecodeWaves);
  static_assert(LT::COPIES % kDecodeWaves == 0 || LT::COPIES < kDecodeWaves, "copy split");
  __shared__ __attribute__((aligned(1024))) char smem_raw[NS * LT::BYTES];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;

  const int k = blockIdx.x;
  const long long lo = range_start(k, a.N, a.G), hi = range_start(k + 1, a.N, a.G);
  if (lo >= hi) return;  // whole workgroup (the host keeps G <= N)
  const int ntiles = (int)((hi - lo + LT::KT - 1) / LT::KT);

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, kq = lane >> 4;
  const int h = 16 * w + l16;
  const bool compute = 16 * w < a.H;  // wave-uniform
  const bool hvalid = h < a.H;
  const int hc = hvalid ? h : a.H - 1;

  // first sequence with rows in [lo, hi): the largest i with cu[i] <= lo
  // First sequence with rows in [lo, hi): the largest i with cu[i] <= lo.
  // Sequence bookkeeping is wave-uniform and fits 32 bits (the host keeps
  // the cache below 2^31 rows), so it lives in scalar registers.
  int i;
  {
    int l = 0, r = a.B - 1;
    while (l < r) {
      const int mid = (l + r + 1) >> 1;
      if ((long long)a.cu[mid] <= lo) l = mid; else r = mid - 1;
    }
    i = __builtin_amdgcn_readfirstlane(l);
  }
  int seq_lo = __builtin_amdgcn_readfirstlane(a.cu[i]), seq_end = __builtin_amdgcn_readfirstlane(a.cu[i + 1]);

  TileCopier<R, kDecodeWaves> copier;
  copier.init(w, lane);
  WaveAttn<R> st;
  auto load_q = [&](int seq) {
    const bf16* src = a.qabs + ((size_t)seq * a.H + hc) * R + 8 * kq;
#pragma unroll
    for (int kk = 0; kk < R / 32; ++kk) st.qT[kk] = *(const bf16x8*)(src + 32 * kk);
  };
  // Tile 0 and the first query are needed first: wait for both before the
  // other prefetches go out, so no query load is still pending when the loop
  // starts (the loop's own waits then only track tile copies).
  copier.issue(a.cache, (int)lo, (int)hi, smem);
  if (compute) load_q(i);
  wait_vmcnt<0>();
#pragma unroll
  for (int p = 1; p < NS - 1; ++p)
    if (p < ntiles) copier.issue(a.cache, (int)(lo + p * LT::KT), (int)hi, smem + p * LT::BYTES);
  st.reset();
  st.init_addressing(l16, kq);

  static_assert(NS == 4, "the waits below assume four stages");
  for (int it = 0; it < ntiles; ++it) {
    // Tile `it` has landed once at most the copies of the younger tiles
    // already issued (it+1, it+2, those that exist) are outstanding.
    const int younger = min(NS - 2, ntiles - 1 - it);
    if (younger >= 2) wait_vmcnt<2 * LPW>();
    else if (younger == 1) wait_vmcnt<LPW>();
    else wait_vmcnt<0>();
    // One barrier per tile: it publishes tile `it` and shows that every wave
    // has finished tile it-1, whose stage the copy of tile it+3 refills.
    wg_barrier();
    // That copy goes out after this wave's first score products of the tile
    // rather than right after the barrier, where all eight waves would queue
    // their copies at once (measured about 2% faster).
    const int nx = it + NS - 1;
    bool copy_due = nx < ntiles;  // wave-uniform
    auto issue_next = [&]() {
      if (copy_due) copier.issue(a.cache, (int)(lo + (long long)nx * LT::KT), (int)hi, smem + (nx % NS) * LT::BYTES);
      copy_due = false;
    };
    const MLA_LDS char* tile = smem + (it % NS) * LT::BYTES;
    const int r0 = (int)lo + it * LT::KT;
    const int r1 = min(r0 + LT::KT, (int)hi);

    // a tile may hold the end of one sequence and the start of the next
    while (true) {
      const int a0 = max(r0, seq_lo);
      const int a1 = min(r1, seq_end);
      if (compute && a0 < a1) {
        f32x4 sa, sb;
        st.scores(tile, sa, sb);
        // visible keys of this tile, as tile-relative offsets [k_lo, k_hi)
        const int k_lo = (int)(a0 - r0), k_hi = (int)(a1 - r0);
        if (k_lo > 0 || k_hi < LT::KT) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int ka = 4 * kq + e, kb = ka + 16;
            if (ka < k_lo || ka >= k_hi) sa[e] = -INFINITY;
            if (kb < k_lo || kb >= k_hi) sb[e] = -INFINITY;
          }
        }
        issue_next();
        st.update(tile, sa, sb);
      }
      issue_next();  // waves without heads, pieces without keys in this tile
      // the piece of sequence i inside this range ends in this tile: emit it
      if (seq_end > r1 && r1 < hi) break;
      if (compute) {
        const int slot = k + i;
        const float l_tot = col_sum(st.l_run);
        if (hvalid) {
          // O^T fragment t holds latent dims 16t + 4kq + e
          bf16* dst = a.part_o + ((size_t)slot * a.H + h) * R + 4 * kq;
#pragma unroll
          for (int t = 0; t < R / 16; ++t) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (bf16)st.oT[t][e];
            *(bf16x4*)(dst + 16 * t) = v;
          }
          if (kq == 0) {
            a.part_ml[((size_t)slot * a.H + h) * 2 + 0] = st.m_run;
            a.part_ml[((size_t)slot * a.H + h) * 2 + 1] = l_tot;
          }
        }
      }
      if (seq_end >= hi || i + 1 >= a.B) break;  // range finished
      // keep the next sequence's query loads after the partial stores
      __builtin_amdgcn_sched_barrier(0);
      ++i;
      seq_lo = seq_end;
      seq_end = __builtin_amdgcn_readfirstlane(a.cu[i + 1]);
      if (compute) load_q(i);
      // Take the wait for the new query here, where the switch happens.  Left
      // pending, the loads stay on the compiler's books across the loop back
      // edge, and it then counts vmcnt down to zero inside every later
      // iteration's score products, draining the tile prefetches each time.
      wait_vmcnt<0>();
      st.reset();
      if (seq_lo >= r1) break;  // the next sequence starts in a later tile
    }
  }
}

// ----------------------------------------------------------------- merge
struct DecodeMergeArgs {
  const bf16* part_o;    // [(G + B), H, R]  unnormalised O, bf16
  const float* part_ml;  // [(G + B), H, 2]
  const int* cu;         // [B + 1]
  const bf16* wuv;       // [H, DV, R]
  const bf16* gate;      // [B, H*DV]
  bf16* out;             // [B, H*DV]
  int B, H, G;
  long long N;
  const int* n_dev;      // if set, N and G are read from n_dev[0] and n_dev[1] (paged decode:
                         // cu holds tile counts, G the number of non-empty ranges)
  const int* krange;     // if set, [B, 2]: the first and last range holding rows of each
                         // sequence (the ranges then come from that table, not from N and G)
};

// index of the range that holds cache row x (every range is non-empty)
__device__ __forceinline__ int range_of(long long x, long long N, long long G) {
  return (int)(((x + 1) * G - 1) / N);
}

// Workgroup (head h, 16 sequences), 8 waves.  Phase 1: wave w merges the
// partials of sequences 2w and 2w+1 of the group (half a wave each, 32 lanes
// over the R latent columns), loading the partials of up to kMergeChunk ranges
// at once, and writes o_lat = O / l (bf16) to LDS.  Phase 2: wave w computes
// v-tiles w, w+8, ... of o^T = W_UV[h] o_lat^T on MFMA (the 16 MFMA columns
// are the group's sequences), gates and stores; the first v-tile's W_UV
// operands and gate values are requested at the end of phase 1, before the
// barrier.  At up to 128 VGPRs two workgroups fit on a CU, so the 384
// workgroups of 64 sequences x 96 heads run in one round.
constexpr int kMergeSeqs = 16;
constexpr int kMergeWaves = 8;
constexpr int kMergeChunk = 8;

template <int DV, int R>
__global__ void __launch_bounds__(64 * kMergeWaves) __attribute__((amdgpu_waves_per_eu(4)))
mla_decode_merge(DecodeMergeArgs a) {
  constexpr int CPL = R / 32;  // latent columns per lane (32 lanes per sequence)
  constexpr int NKK = R / 32;
  constexpr int CV = CPL >= 8 ? 8 : CPL;  // elements per partial load
  constexpr int NL = CPL / CV;            // loads per partial and lane
  static_assert(CPL % CV == 0 && (CV == 1 || CV == 8), "merge split");
  static_assert(kMergeSeqs == 2 * kMergeWaves, "one half wave per sequence");
  using raw_t = std::conditional_t<CV == 8, bf16x8, bf16>;
  __shared__ __attribute__((aligned(16))) bf16 olat[kMergeSeqs][R + 8];

  // 1-D grid of H x nb workgroups (nb = ceil(B / 16)).  With H % 8 == 0 the
  // nb workgroups of head h get ids congruent to h mod 8, i.e. they run on
  // one XCD and read W_UV[h] from HBM once.
  const int nb = (a.B + kMergeSeqs - 1) / kMergeSeqs;
  int h, bb;
  if ((a.H & 7) == 0) {
    const int id = blockIdx.x;
    h = (id / (8 * nb)) * 8 + (id & 7);
    bb = (id >> 3) % nb;
  } else {
    h = blockIdx.x / nb;
    bb = blockIdx.x % nb;
  }
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, kq = lane >> 4;

  // phase 2 operands (MFMA column l16 = sequence bb*16 + l16)
  const int ip = bb * kMergeSeqs + l16;
  const bool pvalid = ip < a.B;
  const int ipc = ip < a.B ? ip : a.B - 1;
  const bf16* wv = a.wuv + (size_t)h * DV * R;
  const size_t orow = (size_t)ipc * a.H * DV + (size_t)h * DV;
  auto load_w = [&](int vt, bf16x8 (&wa)[NKK], bf16x4& gv) {
    const bf16* wrow = wv + (size_t)(16 * vt + l16) * R + 8 * kq;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) wa[kk] = *(const bf16x8*)(wrow + 32 * kk);
    gv = *(const bf16x4*)(a.gate + orow + 16 * vt + 4 * kq);
  };
  bf16x8 wa[NKK];
  bf16x4 gv;

  {
    const long long N = a.n_dev ? (long long)a.n_dev[0] : a.N;
    const long long G = a.n_dev ? (long long)a.n_dev[1] : a.G;
    const int sl = 2 * w + (lane >> 5);  // sequence of this half wave in the group
    const int l32 = lane & 31;
    const int i = bb * kMergeSeqs + sl;
    const int ic = i < a.B ? i : a.B - 1;
    int k0, k1;
    if (a.krange) {
      k0 = a.krange[2 * ic];
      k1 = a.krange[2 * ic + 1];
    } else {
      const long long s0 = a.cu[ic], s1 = a.cu[ic + 1];
      k0 = range_of(s0, N, G);
      k1 = range_of(s1 - 1, N, G);
    }
    const int j0 = CPL * l32;
    float m = -INFINITY, L = 0.0f;
    float acc[CPL];
#pragma unroll
    for (int u = 0; u < CPL; ++u) acc[u] = 0.0f;
    for (int kc = k0; kc <= k1; kc += kMergeChunk) {
      // every partial of the chunk is in flight at once, kept as loaded until used
      float mk[kMergeChunk], lk[kMergeChunk];
      raw_t ok[kMergeChunk][NL];
#pragma unroll
      for (int c = 0; c < kMergeChunk; ++c) {
        const int k = min(kc + c, k1);
        const size_t base = (size_t)(k + ic) * a.H + h;
        const float2 ml = *(const float2*)(a.part_ml + base * 2);
        mk[c] = ml.x;
        lk[c] = ml.y;
        const bf16* src = a.part_o + base * R + j0;
#pragma unroll
        for (int u = 0; u < NL; ++u) ok[c][u] = *(const raw_t*)(src + CV * u);
      }
#pragma unroll
      for (int c = 0; c < kMergeChunk; ++c) {
        if (kc + c > k1) break;  // partials past the last range are repeats
        const float m_new = fmaxf(m, mk[c]);
        const float sa = fast_exp2(m - m_new), sb = fast_exp2(mk[c] - m_new);
        L = L * sa + lk[c] * sb;
#pragma unroll
        for (int u = 0; u < NL; ++u) {
          if constexpr (CV == 8) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[8 * u + e] = acc[8 * u + e] * sa + (float)ok[c][u][e] * sb;
          } else {
            acc[u] = acc[u] * sa + (float)ok[c][u] * sb;
          }
        }
        m = m_new;
      }
    }
    // the first v-tile's operands are requested only now: a wave's loads
    // complete in order, so issued earlier they would delay krange and the
    // partials behind them
    if (w < DV / 16) load_w(w, wa, gv);
    const float invL = 1.0f / L;
#pragma unroll
    for (int u = 0; u < CPL; ++u) olat[sl][j0 + u] = (bf16)(acc[u] * invL);
  }
  __syncthreads();

  // o_lat^T B operand for k-step kk: slot p <-> latent dim 32kk + 8kq + p
  for (int vt = w; vt < DV / 16; vt += kMergeWaves) {
    if (vt != w) load_w(vt, wa, gv);
    f32x4 acc = f32x4{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const bf16x8 bv = *(const bf16x8*)&olat[l16][32 * kk + 8 * kq];
      acc = mfma16(wa[kk], bv, acc);
    }
    if (pvalid) {
      bf16x4 ov;
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[e] = (bf16)(acc[e] * sigmoidf_((float)gv[e]));
      *(bf16x4*)(a.out + orow + 16 * vt + 4 * kq) = ov;
    }
  }
}

// ----------------------------------------------------------------- paged
// Decode against a paged latent cache: sequence i's row u lives in page
// block_table[i, u / page_size] at slot u % page_size of a page pool
// [num_pages, page_size, R].  page_size is a power of two of at least the
// 32-row tile, so a tile never crosses a page.  The split works in tile units: sequence i
// owns ceil(len_i / 32) consecutive tiles of a virtual tile sequence, range
// k of G covers tiles [floor(k NT / G), floor((k+1) NT / G)), and a tile
// belongs to exactly one sequence.  Partial slots, the merge and its
// range arithmetic are those of the packed decode, in tile units.

struct DecodePagedArgs {
  const bf16* qabs;         // [B, H, R]
  const bf16* pages;        // [num_pages, page_size, R]
  const int* block_table;   // [B, max_pages]
  const int* lens;          // [B] clamped lengths (mla_paged_prepare)
  const int* cu_t;          // [B + 2] tile prefix sums, then the range count (mla_paged_prepare)
  bf16* part_o;             // [(G + B), H, R]  unnormalised O, bf16
  float* part_ml;           // [(G + B), H, 2]
  int B, H, G;                           // G: workgroups launched (>= the range count)
  int page_shift, max_pages, num_pages;  // pages of 2^page_shift rows
};

template <int R>
__global__ void __launch_bounds__(64 * kDecodeWaves)
__attribute__((amdgpu_waves_per_eu(2, 2)))
mla_decode_split_paged(DecodePagedArgs a) {
  using LT = LatentTile<R>;
  constexpr int NS = kDecodeStages;
  constexpr int LPW = copies_per_wave<R>(kDecodeWaves);
  static_assert(LT::COPIES % kDecodeWaves == 0 || LT::COPIES < kDecodeWaves, "copy split");
  static_assert(LT::KT == 32, "tile rows");
  __shared__ __attribute__((aligned(1024))) char smem_raw[NS * LT::BYTES];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;

  const int k = blockIdx.x;
  const int NT = __builtin_amdgcn_readfirstlane(a.cu_t[a.B]);
  const int G = __builtin_amdgcn_readfirstlane(a.cu_t[a.B + 1]);  // min(launched, NT): ranges are non-empty
  if (k >= G) return;  // the whole workgroup leaves
  const int lo = (int)((long long)k * NT / G), hi = (int)((long long)(k + 1) * NT / G);
  const int ntiles = hi - lo;

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, kq = lane >> 4;
  const int h = 16 * w + l16;
  const bool compute = 16 * w < a.H;  // wave-uniform
  const bool hvalid = h < a.H;
  const int hc = hvalid ? h : a.H - 1;

  // the sequence of tile lo: the largest i with cu_t[i] <= lo
  int i;
  {
    int l = 0, r = a.B - 1;
    while (l < r) {
      const int mid = (l + r + 1) >> 1;
      if (a.cu_t[mid] <= lo) l = mid; else r = mid - 1;
    }
    i = __builtin_amdgcn_readfirstlane(l);
  }
  int seq_t0 = __builtin_amdgcn_readfirstlane(a.cu_t[i]);
  int seq_t1 = __builtin_amdgcn_readfirstlane(a.cu_t[i + 1]);
  int len = __builtin_amdgcn_readfirstlane(a.lens[i]);

  TileCopier<R, kDecodeWaves> copier;
  copier.init(w, lane);
  // The copy cursor runs NS - 1 tiles ahead of the compute cursor and keeps
  // its own sequence bookkeeping (scalar registers).
  // The page index is looked up once per page and the length once per
  // sequence; every lookup is a scalar load that waits for itself.
  int pi = i, p_t0 = seq_t0, p_t1 = seq_t1, p_len = len;
  int p_page = -1, p_pg = 0;
  auto issue_tile = [&](int t, MLA_LDS char* stage) {
    while (t >= p_t1) {  // every sequence owns at least one tile
      ++pi;
      p_t0 = p_t1;
      p_t1 = sload_i32(a.cu_t + pi + 1);
      p_len = sload_i32(a.lens + pi);
      p_page = -1;
    }
    const int pos = (t - p_t0) * LT::KT;
    if ((pos >> a.page_shift) != p_page) {
      p_page = pos >> a.page_shift;
      p_pg = sload_i32(a.block_table + (size_t)pi * a.max_pages + p_page);
    }
    int pg = p_pg;
    int valid = min(p_len - pos, LT::KT);
    if ((unsigned)pg >= (unsigned)a.num_pages) {
      pg = 0;
      valid = 0;
    }
    const size_t row = ((size_t)pg << a.page_shift) + (pos & ((1 << a.page_shift) - 1));
    copier.issue(a.pages + row * R, 0, valid, stage);
  };

  WaveAttn<R> st;
  auto load_q = [&](int seq) {
    const bf16* src = a.qabs + ((size_t)seq * a.H + hc) * R + 8 * kq;
#pragma unroll
    for (int kk = 0; kk < R / 32; ++kk) st.qT[kk] = *(const bf16x8*)(src + 32 * kk);
  };
  issue_tile(lo, smem);
  if (compute) load_q(i);
  wait_vmcnt<0>();
#pragma unroll
  for (int p = 1; p < NS - 1; ++p)
    if (p < ntiles) issue_tile(lo + p, smem + p * LT::BYTES);
  st.reset();
  st.init_addressing(l16, kq);

  static_assert(NS == 4, "the waits below assume four stages");
  for (int it = 0; it < ntiles; ++it) {
    const int younger = min(NS - 2, ntiles - 1 - it);
    if (younger >= 2) wait_vmcnt<2 * LPW>();
    else if (younger == 1) wait_vmcnt<LPW>();
    else wait_vmcnt<0>();
    wg_barrier();  // tile `it` visible; every wave is done with tile it-1
    // the copy of tile it+3 goes out after the score products, as in the
    // packed kernel
    const int nx = it + NS - 1;
    const MLA_LDS char* tile = smem + (it % NS) * LT::BYTES;
    const int t = lo + it;
    if (t == seq_t1) {
      // the previous tile ended a sequence (its partial is out): start the next
      ++i;
      seq_t0 = seq_t1;
      seq_t1 = sload_i32(a.cu_t + i + 1);
      len = sload_i32(a.lens + i);
      if (compute) load_q(i);
      wait_vmcnt<0>();  // see the packed kernel: no query load stays pending across the back edge
      st.reset();
    }

    if (compute) {
      f32x4 sa, sb;
      st.scores(tile, sa, sb);
      if (nx < ntiles) issue_tile(lo + nx, smem + (nx % NS) * LT::BYTES);
      const int k_hi = len - (t - seq_t0) * LT::KT;  // rows of this sequence in the tile
      if (k_hi < LT::KT) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (4 * kq + e >= k_hi) sa[e] = -INFINITY;
          if (16 + 4 * kq + e >= k_hi) sb[e] = -INFINITY;
        }
      }
      st.update(tile, sa, sb);
      if (t + 1 == seq_t1 || t + 1 == hi) {
        // this range's piece of sequence i ends here: emit its partial
        const int slot = k + i;
        const float l_tot = col_sum(st.l_run);
        if (hvalid) {
          bf16* dst = a.part_o + ((size_t)slot * a.H + h) * R + 4 * kq;
#pragma unroll
          for (int u = 0; u < R / 16; ++u) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (bf16)st.oT[u][e];
            *(bf16x4*)(dst + 16 * u) = v;
          }
          if (kq == 0) {
            a.part_ml[((size_t)slot * a.H + h) * 2 + 0] = st.m_run;
            a.part_ml[((size_t)slot * a.H + h) * 2 + 1] = l_tot;
          }
        }
      }
    } else if (nx < ntiles) {
      issue_tile(lo + nx, smem + (nx % NS) * LT::BYTES);
    }
  }
}

// Cache append: row c_new[i] becomes row positions[i] of sequence i.  One
// wave per row, 16-byte chunks; a position or page index out of range skips
// the row (nothing is written).
__global__ void __launch_bounds__(256) mla_cache_append_paged(const char* __restrict__ c_new,
                                                              char* __restrict__ pages,
                                                              const int* __restrict__ block_table,
                                                              const int* __restrict__ positions, int B,
                                                              int row_bytes, int page_size, int max_pages,
                                                              int num_pages) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (i >= B) return;
  const int u = positions[i];
  if (u < 0 || u >= max_pages * page_size) return;
  const int pg = block_table[(size_t)i * max_pages + u / page_size];
  if (pg < 0 || pg >= num_pages) return;
  const char* src = c_new + (size_t)i * row_bytes;
  char* dst = pages + ((size_t)pg * page_size + u % page_size) * row_bytes;
  for (int off = 16 * lane; off < row_bytes; off += 16 * 64)
    *(u32x4*)(dst + off) = *(const u32x4*)(src + off);
}

}  // namespace mla
