// Host side of the MI355X absorbed Gated MLA library: argument checks,
// workspace carving and kernel launches behind the C ABI of mla_absorb.h.
#include "mla_absorb.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "common.h"
#include "backward_bf16.h"
#include "decode_bf16.h"
#include "decode_solo.h"
#include "f32_kernels.h"
#include "forward_bf16.h"
#include "gemm_bf16.h"
#include "layer_backward_bf16.h"
#include "prefill_bf16.h"
#include "prefill_solo.h"

// Scratch of mla_absorb_decode_noalloc: one static device buffer per GPU
// (each device that loads this code object holds its own copy at its own
// address until the process ends).  Its host-side name is not a device
// address: host code only ever uses the pointer hipGetSymbolAddress returns
// for the current device, resolved once per device and kept below.
static __device__ __align__(256) char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

using mla::bf16;

constexpr size_t kAlign = 256;
constexpr size_t kBadSize = (size_t)-1;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool bf16_shape_supported(int dq, int dv, int r) {
  return (dq == 16 && dv == 16 && r == 32) || (dq == 64 && dv == 64 && r == 256) ||
         (dq == 128 && dv == 128 && r == 512);
}

bool f32_shape_supported(int dq, int dv, int r) { return dq <= 256 && dv <= 256 && r <= 1024; }

// element counts must stay well inside int64 and the grids inside int32
bool fits(long long a, long long b, long long c = 1, long long d = 1) {
  const long double v = (long double)a * b * c * d;
  return v < 4.0e18L;
}

mla_status launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, null until resolved

// The scratch buffer's device address on the current device.
mla_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

struct DecodeLayout {
  size_t qabs = 0, part_o = 0, part_ml = 0, total = 0;
};

DecodeLayout decode_layout(int B, int H, int r, int G) {
  DecodeLayout L;
  size_t off = 0;
  L.qabs = off;
  off = align_up(off + (size_t)B * H * r * sizeof(bf16));
  L.part_o = off;
  off = align_up(off + (size_t)(G + B) * H * r * sizeof(bf16));
  L.part_ml = off;
  off = align_up(off + (size_t)(G + B) * H * 2 * sizeof(float));
  L.total = off;
  return L;
}

// r >= 256: one wave per SIMD owns a head's 32 positions over the whole
// latent; r = 32: one wave per (head, 16 positions).
template <int DQ, int DV, int R, bool PAGED = false>
void launch_prefill_bf16(mla::PrefillArgs a, hipStream_t s) {
  if constexpr (R >= 256) {
    a.ntb = (a.T + mla::kSoloRows - 1) / mla::kSoloRows;
    a.nhg = a.H;  // one head per workgroup
    a.xcd_remap = (a.nhg % 8) == 0 ? 1 : 0;  // the order without a queue
    hipLaunchKernelGGL((mla::mla_prefill_solo_kernel<DQ, DV, R, PAGED>), dim3(a.B * a.ntb * a.nhg),
                       dim3(64 * mla::kSoloWaves), 0, s, a);
  } else {
    a.ntb = (a.T + mla::kPrefillRows - 1) / mla::kPrefillRows;
    a.nhg = (a.H + 3) / 4;
    a.xcd_remap = (a.nhg % 8) == 0 ? 1 : 0;
    hipLaunchKernelGGL((mla::mla_prefill_bf16_kernel<DQ, DV, R, PAGED>), dim3(a.B * a.ntb * a.nhg),
                       dim3(64 * mla::kPrefillWaves), 0, s, a);
  }
}

template <int DQ, int DV, int R>
void launch_decode_bf16(const mla::DecodeAbsorbArgs& aa, const mla::DecodeSplitArgs& sa,
                        const mla::DecodeMergeArgs& ma, hipStream_t s) {
  constexpr int JC = R < 64 ? R : 64;
  hipLaunchKernelGGL((mla::mla_decode_absorb<DQ, R>), dim3(aa.H * (R / JC)), dim3(256), 0, s, aa);
  hipLaunchKernelGGL((mla::mla_decode_split<R>), dim3(sa.G), dim3(64 * mla::kDecodeWaves), 0, s, sa);
  hipLaunchKernelGGL((mla::mla_decode_merge<DV, R>), dim3(((ma.B + mla::kMergeSeqs - 1) / mla::kMergeSeqs) * ma.H),
                     dim3(64 * mla::kMergeWaves), 0, s, ma);
}

template <int DQ, int DV, int R>
void launch_decode_paged_bf16(const mla::DecodeAbsorbArgs& aa, const int* seq_lens, int max_rows,
                              const mla::DecodePagedArgs& sa, const mla::DecodeMergeArgs& ma, hipStream_t s) {
  constexpr int JC = R < 64 ? R : 64;
  mla::PrepareArgs pa{seq_lens, nullptr, sa.B, max_rows, sa.G, const_cast<int*>(sa.lens), const_cast<int*>(sa.cu_t),
                      nullptr, nullptr, 0};
  hipLaunchKernelGGL(mla::mla_paged_prepare, dim3(1), dim3(256), 0, s, pa);
  hipLaunchKernelGGL((mla::mla_decode_absorb<DQ, R>), dim3(aa.H * (R / JC)), dim3(256), 0, s, aa);
  hipLaunchKernelGGL((mla::mla_decode_split_paged<R>), dim3(sa.G), dim3(64 * mla::kDecodeWaves), 0, s, sa);
  hipLaunchKernelGGL((mla::mla_decode_merge<DV, R>), dim3(((ma.B + mla::kMergeSeqs - 1) / mla::kMergeSeqs) * ma.H),
                     dim3(64 * mla::kMergeWaves), 0, s, ma);
}

// r = 512: per-sequence tiles, one-wave-per-SIMD split kernel (packed cache:
// cu != nullptr, paged: seq_lens != nullptr); the merge takes its ranges in
// tile units from the prepared prefix sums.
template <int DQ, int DV, int R, bool PAGED>
void launch_decode_solo(mla::DecodeAbsorbArgs aa, const int* seq_lens, const int* cu, int max_rows, int G,
                        int* krange, const mla::DecodeSoloArgs& sa, mla::DecodeMergeArgs ma, hipStream_t s) {
  constexpr int JC = R < 64 ? R : 64;
  // the absorb's first workgroup prepares the tile sums and the range table
  aa.with_prep = 1;
  aa.prep = mla::PrepareArgs{seq_lens, cu, sa.B, max_rows, G, const_cast<int*>(sa.lens), const_cast<int*>(sa.cu_t),
                             const_cast<int*>(sa.rt), krange, mla::kDecodeSwitchTiles};
  hipLaunchKernelGGL((mla::mla_decode_absorb<DQ, R>), dim3(aa.H * (R / JC) + 1), dim3(256), 0, s, aa);
  if (sa.H <= 3 * 32)
    hipLaunchKernelGGL((mla::mla_decode_solo<R, PAGED, true>), dim3(G), dim3(64 * mla::kDecodeSoloWaves), 0, s, sa);
  else
    hipLaunchKernelGGL((mla::mla_decode_solo<R, PAGED, false>), dim3(G), dim3(64 * mla::kDecodeSoloWaves), 0, s, sa);
  ma.cu = sa.cu_t;
  ma.n_dev = sa.cu_t + sa.B;
  ma.N = 0;
  ma.krange = krange;
  hipLaunchKernelGGL((mla::mla_decode_merge<DV, R>), dim3(((ma.B + mla::kMergeSeqs - 1) / mla::kMergeSeqs) * ma.H),
                     dim3(64 * mla::kMergeWaves), 0, s, ma);
}

struct PagedDecodeLayout {
  DecodeLayout d;
  size_t lens = 0, cu_t = 0, rt = 0, krange = 0, total = 0;
};

PagedDecodeLayout paged_decode_layout(int B, int H, int r, int G) {
  PagedDecodeLayout L;
  L.d = decode_layout(B, H, r, G);
  size_t off = L.d.total;
  L.lens = off;
  off = align_up(off + (size_t)B * sizeof(int));
  L.cu_t = off;
  off = align_up(off + (size_t)(B + 2) * sizeof(int));
  L.rt = off;
  off = align_up(off + (size_t)(G + 1) * sizeof(int));
  L.krange = off;
  off = align_up(off + (size_t)B * 2 * sizeof(int));
  L.total = off;
  return L;
}

// page pool geometry shared by the paged entry points: log2 of a positive
// power of two, -1 for anything else (no loop, no shift past bit 30)
int log2_exact(int v) {
  if (v <= 0 || (v & (v - 1)) != 0) return -1;
  return __builtin_ctz((unsigned)v);
}

bool paged_geometry_ok(int B, int r, long long num_pages, int page_size, int max_pages) {
  if (num_pages <= 0 || page_size < 32 || max_pages <= 0 || log2_exact(page_size) < 0) return false;
  return num_pages < (1LL << 31) && fits(num_pages, page_size, r) &&
         (long long)max_pages * page_size < (1LL << 31) && fits(B, max_pages) &&
         (long long)B * max_pages * page_size / 32 < (1LL << 31);
}

void launch_wuk_transpose(const bf16* w, bf16* wt, int H, int dq, int r, hipStream_t s,
                          unsigned* queue = nullptr) {
  hipLaunchKernelGGL((mla::mla_wuk_transpose<bf16>), dim3((r + 31) / 32, (dq + 31) / 32, H), dim3(256), 0, s,
                     w, wt, dq, r, queue);
}

// Prefill workspace: W_UK^T [H, r, d_q] bf16, then the work-item counter of
// the r >= 256 kernel in a slot of its own.
size_t prefill_ws_bytes(int H, int r, int dq) {
  return align_up((size_t)H * r * dq * sizeof(bf16)) + kAlign;
}

struct ForwardLayout {
  size_t c = 0, ql = 0, q = 0, gate = 0, o = 0, core = 0, total = 0;
};

// Workspace of the full forward: the latent, the normalised query latent, q,
// the gate pre-activations, the gated core output and the core's own workspace.
ForwardLayout forward_layout(int B, int T, int q_rank, int H, int dq, int dv, int r) {
  const size_t N = (size_t)B * T;
  ForwardLayout L;
  size_t off = 0;
  L.c = off;    off = align_up(off + N * r * sizeof(bf16));
  L.ql = off;   off = align_up(off + N * q_rank * sizeof(bf16));
  L.q = off;    off = align_up(off + N * H * dq * sizeof(bf16));
  L.gate = off; off = align_up(off + N * H * dv * sizeof(bf16));
  L.o = off;    off = align_up(off + N * H * dv * sizeof(bf16));
  L.core = off; off = align_up(off + prefill_ws_bytes(H, r, dq));
  L.total = off;
  return L;
}

// Y[z] = alpha X[z] W[z]^T for z < batch, every operand strided.  The
// 256 x 256 tile when it still gives at least one workgroup per CU (256),
// else 128 x 128.
void launch_gemm_batched(const bf16* x, int lda, long long bsx, const bf16* w, int ldw, long long bsw, bf16* y, int ldy,
                         long long bsy, int M, int N, int K, float alpha, int batch, hipStream_t s) {
  mla::GemmArgs g{};
  g.x = x; g.w = w; g.y = y; g.M = M; g.N = N; g.K = K; g.lda = lda; g.ldw = ldw; g.ldy = ldy;
  g.bsx = bsx; g.bsw = bsw; g.bsy = bsy; g.alpha = alpha;
  const long long big = (long long)((N + mla::kGemmBig - 1) / mla::kGemmBig) *
                        ((M + mla::kGemmBig - 1) / mla::kGemmBig) * batch;
  if (big >= 256) {
    g.tiles_n = (N + mla::kGemmBig - 1) / mla::kGemmBig;
    hipLaunchKernelGGL(mla::mla_gemm_nt_big, dim3((unsigned)(big / batch), batch), dim3(512), 0, s, g);
  } else {
    g.tiles_n = (N + mla::kGemmTile - 1) / mla::kGemmTile;
    const long long grid = (long long)g.tiles_n * ((M + mla::kGemmTile - 1) / mla::kGemmTile);
    hipLaunchKernelGGL(mla::mla_gemm_nt, dim3((unsigned)grid, batch), dim3(256), 0, s, g);
  }
}

// Y = X W^T, every operand dense row-major (one batch)
void launch_gemm(const bf16* x, const bf16* w, bf16* y, int M, int N, int K, hipStream_t s) {
  launch_gemm_batched(x, K, 0, w, K, 0, y, N, 0, M, N, K, 1.0f, 1, s);
}

// y = RMSNorm(x) * gain row by row (y may be x); rstd (or null) receives 1/rms
void launch_rmsnorm(const bf16* x, bf16* y, const bf16* gain, float* rstd, int rows, int n, float eps,
                    hipStream_t s) {
  mla::RmsNormArgs a{};
  a.x = x; a.y = y; a.gain = gain; a.rstd = rstd; a.rows = rows; a.n = n; a.eps = eps;
  hipLaunchKernelGGL(mla::mla_rmsnorm_rows, dim3((rows + 3) / 4), dim3(256), 0, s, a);
}

struct BackwardLayout {
  size_t wukT = 0, wuvT = 0, dov = 0, ld = 0, qabs = 0, dolat = 0, da = 0, dv = 0, part = 0, total = 0;
  int nhg = 0, hpg = 0;
};

BackwardLayout backward_layout(int B, int T, int H, int dq, int dv, int r) {
  BackwardLayout L;
  const size_t BT = (size_t)B * T;
  // at most 8 head groups, none of them empty
  L.hpg = (H + 7) / 8;
  L.nhg = (H + L.hpg - 1) / L.hpg;
  size_t off = 0;
  L.wukT = off;  off = align_up(off + (size_t)H * r * dq * sizeof(bf16));
  L.wuvT = off;  off = align_up(off + (size_t)H * r * dv * sizeof(bf16));
  L.dov = off;   off = align_up(off + BT * H * dv * sizeof(bf16));
  L.ld = off;    off = align_up(off + (size_t)H * BT * 2 * sizeof(float));
  L.qabs = off;  off = align_up(off + (size_t)H * BT * r * sizeof(bf16));
  L.dolat = off; off = align_up(off + (size_t)H * BT * r * sizeof(bf16));
  L.da = off;    off = align_up(off + (size_t)H * BT * r * sizeof(bf16));
  L.dv = off;    off = align_up(off + (size_t)H * BT * dv * sizeof(bf16));
  L.part = off;  off = align_up(off + (size_t)L.nhg * BT * r * sizeof(float));
  L.total = off;
  return L;
}

// C[z] = A[z]^T B[z] over K token rows (weight gradients, fp32 out)
void launch_gemm_tn(const bf16* A, size_t a_bytes, int lda, long long bsa, const bf16* Bm, size_t b_bytes, int ldb,
                    long long bsb, float* C, long long bsc, int M, int N, int K, int batch, hipStream_t s) {
  mla::GemmTNArgs g{};
  g.a = A; g.b = Bm; g.c = C; g.M = M; g.N = N; g.K = K; g.lda = lda; g.ldb = ldb;
  g.bsa = bsa; g.bsb = bsb; g.bsc = bsc;
  g.a_bytes = (unsigned)a_bytes; g.b_bytes = (unsigned)b_bytes;
  // the 256 x 256 tile when it still gives at least one workgroup per CU
  const long long big = (long long)((N + mla::kGemmBig - 1) / mla::kGemmBig) *
                        ((M + mla::kGemmBig - 1) / mla::kGemmBig) * batch;
  if (big >= 256) {
    g.tiles_n = (N + mla::kGemmBig - 1) / mla::kGemmBig;
    hipLaunchKernelGGL(mla::mla_gemm_tn_big, dim3((unsigned)(big / batch), batch), dim3(512), 0, s, g);
    return;
  }
  g.tiles_n = (N + mla::kGemmTile - 1) / mla::kGemmTile;
  const int tiles = g.tiles_n * ((M + mla::kGemmTile - 1) / mla::kGemmTile);
  hipLaunchKernelGGL(mla::mla_gemm_tn, dim3(tiles, batch), dim3(256), 0, s, g);
}

// q_abs2[h] = scale log2e q[:, h, :] W_UK[h] and dol[h] = do[h] W_UV[h], as GEMMs
// against the transposed weights (head-major outputs)
void launch_backward_projections(const bf16* q, const bf16* wukT, const bf16* dov, const bf16* wuvT, bf16* qabs,
                                 bf16* dolat, int BT, int H, int dq, int dv, int r, float qscale, hipStream_t s) {
  launch_gemm_batched(q, H * dq, dq, wukT, dq, (long long)r * dq, qabs, r, (long long)BT * r, BT, r, dq, qscale, H,
                      s);
  launch_gemm_batched(dov, dv, (long long)BT * dv, wuvT, dv, (long long)r * dv, dolat, r, (long long)BT * r, BT, r, dv,
                      1.0f, H, s);
}

template <int DQ, int DV, int R>
void launch_backward_bf16(const mla::BwdPrepArgs& pa, const mla::BwdArgs& ba, const bf16* q, const bf16* wukT,
                          const bf16* wuvT, hipStream_t s) {
  hipLaunchKernelGGL(mla::mla_bwd_prep<DV>, dim3(pa.B * pa.T), dim3(256), 0, s, pa);
  launch_backward_projections(q, wukT, pa.dov, wuvT, const_cast<bf16*>(ba.qabs), const_cast<bf16*>(ba.dolat),
                              pa.B * pa.T, ba.H, DQ, DV, R, ba.scale * mla::kLog2e, s);
  hipLaunchKernelGGL((mla::mla_bwd_query<R>), dim3(ba.B * ba.ntb * ba.H), dim3(64 * mla::kBwdWaves), 0, s, ba);
  const int nkb = (ba.T + mla::kBwdKeys - 1) / mla::kBwdKeys;
  hipLaunchKernelGGL((mla::mla_bwd_key<DV, R>), dim3(ba.B * nkb * ba.nhg), dim3(64 * mla::kBwdWaves), 0, s, ba);
}

// Varlen: the prepare kernel, then the paged prefill kernels over its block
// list (max_blocks = ceil(Nq / rows per block) + B workgroups per head group).
template <int DQ, int DV, int R>
void launch_varlen_bf16(mla::PrefillArgs a, const int* cu_q, const int* seq_lens, int Nq, int max_rows,
                        hipStream_t s) {
  constexpr int BR = R >= 256 ? mla::kSoloRows : mla::kPrefillRows;
  const int max_blocks = (Nq + BR - 1) / BR + a.B;
  hipLaunchKernelGGL(mla::mla_varlen_prepare, dim3(1), dim3(256), 0, s, cu_q, seq_lens, a.B, Nq, max_rows, BR,
                     max_blocks, const_cast<int4*>(a.seq), const_cast<int2*>(a.blocks), const_cast<int*>(a.nblocks));
  if constexpr (R >= 256) {
    a.nhg = a.H;  // one head per workgroup
    a.xcd_remap = 0;
    hipLaunchKernelGGL((mla::mla_prefill_solo_kernel<DQ, DV, R, true, true>), dim3(max_blocks * a.nhg),
                       dim3(64 * mla::kSoloWaves), 0, s, a);
  } else {
    a.nhg = (a.H + 3) / 4;
    a.xcd_remap = 0;
    hipLaunchKernelGGL((mla::mla_prefill_bf16_kernel<DQ, DV, R, true, true>), dim3(max_blocks * a.nhg),
                       dim3(64 * mla::kPrefillWaves), 0, s, a);
  }
}

// Saved state of a training forward of the full layer: what the backward
// reads (the norms' inputs and 1/rms, their outputs, q, the gate, the gated
// core output and the core's log-sum-exp) plus the core's own workspace.
struct TrainLayout {
  size_t c_pre = 0, c = 0, rstd_c = 0, ql_pre = 0, ql = 0, rstd_q = 0, q = 0, gate = 0, o = 0, lse = 0, core = 0,
         total = 0;
};

TrainLayout train_layout(int B, int T, int q_rank, int H, int dq, int dv, int r) {
  const size_t N = (size_t)B * T;
  TrainLayout L;
  size_t off = 0;
  L.c_pre = off;  off = align_up(off + N * r * sizeof(bf16));
  L.c = off;      off = align_up(off + N * r * sizeof(bf16));
  L.rstd_c = off; off = align_up(off + N * sizeof(float));
  L.ql_pre = off; off = align_up(off + N * q_rank * sizeof(bf16));
  L.ql = off;     off = align_up(off + N * q_rank * sizeof(bf16));
  L.rstd_q = off; off = align_up(off + N * sizeof(float));
  L.q = off;      off = align_up(off + N * H * dq * sizeof(bf16));
  L.gate = off;   off = align_up(off + N * H * dv * sizeof(bf16));
  L.o = off;      off = align_up(off + N * H * dv * sizeof(bf16));
  L.lse = off;    off = align_up(off + N * H * sizeof(float));
  L.core = off;   off = align_up(off + prefill_ws_bytes(H, r, dq));
  L.total = off;
  return L;
}

constexpr int kNormBwdGroups = 256;  // workgroups of the RMSNorm backward (partial rows of the gain gradient)

// Workspace of the layer backward.  gcat [N, Kc] holds, side by side, the
// gradients of the three products of x (gate pre-activations, query and
// latent down-projections before their norms), Kc = H dv + q_rank + r, so
// that dx is one product with the matching transposed weights wcatT [D, Kc].
struct LayerBwdLayout {
  size_t gcat = 0, dout = 0, dq = 0, dc = 0, dql = 0, woT = 0, wqupT = 0, wcatT = 0, part = 0, core = 0, total = 0;
  int Kc = 0;
};

LayerBwdLayout layer_bwd_layout(int B, int T, int D, int q_rank, int H, int dq, int dv, int r) {
  const size_t N = (size_t)B * T;
  LayerBwdLayout L;
  L.Kc = H * dv + q_rank + r;
  size_t off = 0;
  L.gcat = off;  off = align_up(off + N * L.Kc * sizeof(bf16));
  L.dout = off;  off = align_up(off + N * H * dv * sizeof(bf16));
  L.dq = off;    off = align_up(off + N * H * dq * sizeof(bf16));
  L.dc = off;    off = align_up(off + N * r * sizeof(bf16));
  L.dql = off;   off = align_up(off + N * q_rank * sizeof(bf16));
  L.woT = off;   off = align_up(off + (size_t)H * dv * D * sizeof(bf16));
  L.wqupT = off; off = align_up(off + (size_t)q_rank * H * dq * sizeof(bf16));
  L.wcatT = off; off = align_up(off + (size_t)D * L.Kc * sizeof(bf16));
  L.part = off;  off = align_up(off + (size_t)kNormBwdGroups * (q_rank > r ? q_rank : r) * sizeof(float));
  L.core = off;  off = align_up(off + backward_layout(B, T, H, dq, dv, r).total);
  L.total = off;
  return L;
}

// dst[:, col0 + i] = src[i, :]^T for src [rows, cols]: dst rows ld_dst apart
void launch_transpose_into(const bf16* src, int rows, int cols, bf16* dst, long long ld_dst, hipStream_t s) {
  hipLaunchKernelGGL(mla::mla_transpose_into, dim3((cols + 31) / 32, (rows + 31) / 32), dim3(256), 0, s, src, rows,
                     cols, dst, ld_dst);
}

// RMSNorm backward of rows [rows, n] and the gain gradient dgain [n]
void launch_rmsnorm_backward(const bf16* du, int ld_du, const bf16* v, const float* rstd, const bf16* gain, bf16* dv,
                             int ld_dv, float* part, float* dgain, int rows, int n, hipStream_t s) {
  mla::RmsNormBwdArgs a{};
  a.du = du; a.v = v; a.rstd = rstd; a.gain = gain; a.dv = dv; a.part = part;
  a.rows = rows; a.n = n; a.ld_du = ld_du; a.ld_dv = ld_dv;
  const int groups = (rows + 3) / 4 < kNormBwdGroups ? (rows + 3) / 4 : kNormBwdGroups;
  hipLaunchKernelGGL(mla::mla_rmsnorm_backward, dim3(groups), dim3(256), 0, s, a);
  hipLaunchKernelGGL(mla::mla_colsum_f32, dim3((n + 255) / 256), dim3(256), 0, s, part, groups, n, dgain);
}

size_t varlen_meta_bytes(int B, int Nq) {
  const int max_blocks = (Nq + mla::kPrefillRows - 1) / mla::kPrefillRows + B;  // the larger count (16-row blocks)
  return align_up((size_t)B * sizeof(int4)) + align_up((size_t)max_blocks * sizeof(int2)) + align_up(sizeof(int));
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: null or misaligned pointer, non-positive size or non-finite scale";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: shape or dtype outside the compiled set";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace smaller than required";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: the HIP runtime reported a launch error";
  }
  return "MLA_ERR_UNKNOWN";
}

size_t mla_absorb_prefill_workspace_size(int B, int T, int H, int d_q, int r, mla_dtype dtype) {
  if (B <= 0 || T <= 0 || H <= 0 || d_q <= 0 || r <= 0) return kBadSize;
  if (dtype == MLA_DTYPE_F32) return 0;
  if (dtype != MLA_DTYPE_BF16) return kBadSize;
  return prefill_ws_bytes(H, r, d_q);
}

mla_status mla_absorb_prefill(const void* q, const void* c, const void* w_uk, const void* w_uv,
                              const void* gate, void* out, int B, int T, int H, int d_q, int d_v,
                              int r, float scale, mla_dtype dtype, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return mla_absorb_extend(q, c, w_uk, w_uv, gate, out, B, T, T, H, d_q, d_v, r, scale, dtype, workspace,
                           workspace_bytes, stream);
}

// Chunked prefill over a contiguous latent [B, S, r] (block_table null) or a
// paged one (pool c of num_pages pages, geometry checked by the caller).
static mla_status extend_impl(const void* q, const void* c, const int32_t* block_table, long long num_pages,
                       int page_size, int max_pages, const void* w_uk, const void* w_uv, const void* gate,
                       void* out, float* lse, int B, int T, int S, int H, int d_q, int d_v, int r, float scale,
                       mla_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !c || !w_uk || !w_uv || !gate || !out) return MLA_ERR_INVALID_ARG;
  if (B <= 0 || T <= 0 || S < T || H <= 0 || d_q <= 0 || d_v <= 0 || r <= 0) return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(c) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(gate) ||
      !aligned16(out))
    return MLA_ERR_INVALID_ARG;
  if (dtype != MLA_DTYPE_F32 && dtype != MLA_DTYPE_BF16) return MLA_ERR_INVALID_ARG;
  if (!fits(B, T, H, d_q > d_v ? (d_q > r ? d_q : r) : (d_v > r ? d_v : r)) || !fits(B, S, r))
    return MLA_ERR_UNSUPPORTED;
  const bool paged = block_table != nullptr;
  hipStream_t s = (hipStream_t)stream;

  if (dtype == MLA_DTYPE_F32) {
    if (!f32_shape_supported(d_q, d_v, r)) return MLA_ERR_UNSUPPORTED;
    if ((long long)B * T >= (1LL << 31) || H > 65535) return MLA_ERR_UNSUPPORTED;
    mla::F32Args a{};
    a.q = (const float*)q; a.c = (const float*)c; a.cu = nullptr;
    a.wuk = (const float*)w_uk; a.wuv = (const float*)w_uv; a.gate = (const float*)gate;
    a.out = (float*)out;
    a.B = B; a.T = T; a.S = S; a.H = H; a.DQ = d_q; a.DV = d_v; a.R = r; a.N = 0; a.scale = scale;
    a.decode = 0;
    hipLaunchKernelGGL(mla::mla_f32_kernel, dim3(B * T, H), dim3(64), 0, s, a);
    return launch_status();
  }

  if (!bf16_shape_supported(d_q, d_v, r)) return MLA_ERR_UNSUPPORTED;
  const size_t need = mla_absorb_prefill_workspace_size(B, T, H, d_q, r, dtype);
  if (!workspace || !aligned16(workspace)) return need ? MLA_ERR_WORKSPACE : MLA_ERR_INVALID_ARG;
  if (workspace_bytes < need) return MLA_ERR_WORKSPACE;
  // grid bound for the smaller of the two workgroup shapes (16 positions x 4 heads)
  if ((long long)B * ((T + 15) / 16) * ((H + 1) / 2) >= (1LL << 31)) return MLA_ERR_UNSUPPORTED;

  bf16* wukT = (bf16*)workspace;
  unsigned* queue = (unsigned*)((char*)workspace + align_up((size_t)H * r * d_q * sizeof(bf16)));
  launch_wuk_transpose((const bf16*)w_uk, wukT, H, d_q, r, s, queue);

  mla::PrefillArgs a{};
  a.queue = queue;
  a.q = (const bf16*)q; a.c = (const bf16*)c; a.wukT = wukT; a.wuv = (const bf16*)w_uv;
  a.gate = (const bf16*)gate; a.out = (bf16*)out;
  a.B = B; a.T = T; a.S = S; a.H = H;
  a.qscale = scale * mla::kLog2e;
  a.block_table = block_table; a.max_pages = max_pages; a.num_pages = (int)num_pages;
  a.page_shift = paged ? log2_exact(page_size) : 0;
  a.lse = lse;
  if (paged) {
    if (d_q == 16) launch_prefill_bf16<16, 16, 32, true>(a, s);
    else if (d_q == 64) launch_prefill_bf16<64, 64, 256, true>(a, s);
    else launch_prefill_bf16<128, 128, 512, true>(a, s);
  } else {
    if (d_q == 16) launch_prefill_bf16<16, 16, 32>(a, s);
    else if (d_q == 64) launch_prefill_bf16<64, 64, 256>(a, s);
    else launch_prefill_bf16<128, 128, 512>(a, s);
  }
  return launch_status();
}


mla_status mla_absorb_extend(const void* q, const void* c, const void* w_uk, const void* w_uv,
                             const void* gate, void* out, int B, int T, int S, int H, int d_q, int d_v,
                             int r, float scale, mla_dtype dtype, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return extend_impl(q, c, nullptr, 0, 0, 0, w_uk, w_uv, gate, out, nullptr, B, T, S, H, d_q, d_v, r, scale, dtype,
                     workspace, workspace_bytes, stream);
}

mla_status mla_absorb_prefill_train(const void* q, const void* c, const void* w_uk, const void* w_uv,
                                    const void* gate, void* out, float* lse, int B, int T, int H, int d_q, int d_v,
                                    int r, float scale, mla_dtype dtype, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  if (!lse || !aligned16(lse)) return MLA_ERR_INVALID_ARG;
  if (dtype != MLA_DTYPE_BF16) return dtype == MLA_DTYPE_F32 ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  if (!fits(B, H, T)) return MLA_ERR_UNSUPPORTED;
  return extend_impl(q, c, nullptr, 0, 0, 0, w_uk, w_uv, gate, out, lse, B, T, T, H, d_q, d_v, r, scale, dtype,
                     workspace, workspace_bytes, stream);
}

mla_status mla_absorb_extend_paged(const void* q, const void* c_pages, const int32_t* block_table,
                                   const void* w_uk, const void* w_uv, const void* gate, void* out, int B, int T,
                                   int S, int H, int d_q, int d_v, int r, int64_t num_pages, int page_size,
                                   int max_pages, float scale, mla_dtype dtype, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (!c_pages || !block_table || !aligned16(block_table)) return MLA_ERR_INVALID_ARG;
  if (num_pages <= 0 || page_size <= 0 || max_pages <= 0) return MLA_ERR_INVALID_ARG;
  if (page_size < 32 || log2_exact(page_size) < 0 || (long long)max_pages * page_size < S)
    return MLA_ERR_INVALID_ARG;
  if (dtype != MLA_DTYPE_BF16) return dtype == MLA_DTYPE_F32 ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  if (!paged_geometry_ok(B, r, num_pages, page_size, max_pages)) return MLA_ERR_UNSUPPORTED;
  return extend_impl(q, c_pages, block_table, num_pages, page_size, max_pages, w_uk, w_uv, gate, out, nullptr, B, T,
                     S, H, d_q, d_v, r, scale, dtype, workspace, workspace_bytes, stream);
}

size_t mla_absorb_extend_varlen_workspace_size(int B, int Nq, int H, int d_q, int r, mla_dtype dtype) {
  if (B <= 0 || Nq <= 0 || H <= 0 || d_q <= 0 || r <= 0 || dtype != MLA_DTYPE_BF16) return kBadSize;
  return align_up((size_t)H * r * d_q * sizeof(bf16)) + varlen_meta_bytes(B, Nq);
}

mla_status mla_absorb_extend_varlen_paged(const void* q, const void* c_pages, const int32_t* block_table,
                                          const int32_t* cu_q, const int32_t* seq_lens, const void* w_uk,
                                          const void* w_uv, const void* gate, void* out, int B, int Nq, int H, int d_q,
                                          int d_v, int r, int64_t num_pages, int page_size, int max_pages, float scale,
                                          mla_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  const void* ptrs[] = {q, c_pages, block_table, cu_q, seq_lens, w_uk, w_uv, gate, out};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return MLA_ERR_INVALID_ARG;
  if (B <= 0 || Nq <= 0 || H <= 0 || d_q <= 0 || d_v <= 0 || r <= 0) return MLA_ERR_INVALID_ARG;
  if (num_pages <= 0 || max_pages <= 0 || page_size < 32 || log2_exact(page_size) < 0) return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return MLA_ERR_INVALID_ARG;
  if (dtype != MLA_DTYPE_BF16) return dtype == MLA_DTYPE_F32 ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  if (!bf16_shape_supported(d_q, d_v, r)) return MLA_ERR_UNSUPPORTED;
  if (!paged_geometry_ok(B, r, num_pages, page_size, max_pages) || !fits(Nq, H, d_q > d_v ? d_q : d_v))
    return MLA_ERR_UNSUPPORTED;
  if (((long long)Nq / 16 + B) * ((H + 1) / 2) >= (1LL << 31)) return MLA_ERR_UNSUPPORTED;
  const size_t wt = align_up((size_t)H * r * d_q * sizeof(bf16));
  const size_t need = wt + varlen_meta_bytes(B, Nq);
  if (!workspace || !aligned16(workspace)) return MLA_ERR_WORKSPACE;
  if (workspace_bytes < need) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  bf16* wukT = (bf16*)ws;
  launch_wuk_transpose((const bf16*)w_uk, wukT, H, d_q, r, s);

  mla::PrefillArgs a{};
  a.q = (const bf16*)q; a.c = (const bf16*)c_pages; a.wukT = wukT; a.wuv = (const bf16*)w_uv;
  a.gate = (const bf16*)gate; a.out = (bf16*)out;
  a.B = B; a.T = 0; a.S = 0; a.H = H;
  a.qscale = scale * mla::kLog2e;
  a.block_table = block_table; a.max_pages = max_pages; a.num_pages = (int)num_pages;
  a.page_shift = log2_exact(page_size);
  size_t off = wt;
  a.seq = (const int4*)(ws + off);
  off += align_up((size_t)B * sizeof(int4));
  a.blocks = (const int2*)(ws + off);
  off += align_up((size_t)((Nq + mla::kPrefillRows - 1) / mla::kPrefillRows + B) * sizeof(int2));
  a.nblocks = (const int*)(ws + off);
  const int max_rows = max_pages * page_size;
  if (d_q == 16) launch_varlen_bf16<16, 16, 32>(a, cu_q, seq_lens, Nq, max_rows, s);
  else if (d_q == 64) launch_varlen_bf16<64, 64, 256>(a, cu_q, seq_lens, Nq, max_rows, s);
  else launch_varlen_bf16<128, 128, 512>(a, cu_q, seq_lens, Nq, max_rows, s);
  return launch_status();
}

size_t mla_absorb_workspace_size(int is_decode, int B, int T_or_max_len, int H, int r, mla_dtype dtype) {
  if (B <= 0 || T_or_max_len <= 0 || H <= 0 || r <= 0) return kBadSize;
  if (dtype == MLA_DTYPE_F32) return 0;
  if (dtype != MLA_DTYPE_BF16) return kBadSize;
  // the compiled bf16 set pairs each latent width with one head width
  const int d_q = r == 32 ? 16 : r == 256 ? 64 : r == 512 ? 128 : 0;
  if (d_q == 0) return kBadSize;
  return is_decode ? mla_absorb_decode_workspace_size(B, H, d_q, r, 0, dtype)
                   : mla_absorb_prefill_workspace_size(B, T_or_max_len, H, d_q, r, dtype);
}

size_t mla_absorb_decode_workspace_size(int B, int H, int d_q, int r, int num_splits, mla_dtype dtype) {
  if (B <= 0 || H <= 0 || d_q <= 0 || r <= 0) return kBadSize;
  if (dtype == MLA_DTYPE_F32) return 0;
  if (dtype != MLA_DTYPE_BF16) return kBadSize;
  int G = num_splits > 0 ? num_splits : device_cu_count();
  if (G <= 0) return kBadSize;
  return paged_decode_layout(B, H, r, G).total;
}

// Decode over a packed cache with the scratch in the caller's workspace, or
// (noalloc) in the library's static scratch buffer of the current device.
static mla_status decode_impl(const void* q, const void* c_cache, const int32_t* cu_seqlens,
                              const void* w_uk, const void* w_uv, const void* gate, void* out,
                              int B, int H, int d_q, int d_v, int r, int64_t total_len, float scale,
                              int num_splits, mla_dtype dtype, void* workspace,
                              size_t workspace_bytes, void* stream, bool noalloc) {
  if (!q || !c_cache || !cu_seqlens || !w_uk || !w_uv || !gate || !out) return MLA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || d_q <= 0 || d_v <= 0 || r <= 0 || total_len < B) return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(c_cache) || !aligned16(cu_seqlens) || !aligned16(w_uk) ||
      !aligned16(w_uv) || !aligned16(gate) || !aligned16(out))
    return MLA_ERR_INVALID_ARG;
  if (dtype != MLA_DTYPE_F32 && dtype != MLA_DTYPE_BF16) return MLA_ERR_INVALID_ARG;
  if (total_len >= (1LL << 31) || !fits(total_len, r) || !fits(B, H, d_q > d_v ? d_q : d_v))
    return MLA_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;

  if (dtype == MLA_DTYPE_F32) {
    if (!f32_shape_supported(d_q, d_v, r) || H > 65535) return MLA_ERR_UNSUPPORTED;
    mla::F32Args a{};
    a.q = (const float*)q; a.c = (const float*)c_cache; a.cu = cu_seqlens;
    a.wuk = (const float*)w_uk; a.wuv = (const float*)w_uv; a.gate = (const float*)gate;
    a.out = (float*)out;
    a.B = B; a.T = 1; a.H = H; a.DQ = d_q; a.DV = d_v; a.R = r; a.N = total_len;
    a.scale = scale; a.decode = 1;
    hipLaunchKernelGGL(mla::mla_f32_kernel, dim3(B, H), dim3(64), 0, s, a);
    return launch_status();
  }

  if (!bf16_shape_supported(d_q, d_v, r)) return MLA_ERR_UNSUPPORTED;
  if (H > 16 * mla::kDecodeWaves) return MLA_ERR_UNSUPPORTED;  // 16 heads per wave
  int G = num_splits > 0 ? num_splits : device_cu_count();
  if (G <= 0) return MLA_ERR_HIP;
  // the tile prefix sums of the r = 512 path live after the split scratch
  const size_t need = paged_decode_layout(B, H, r, G).total;
  if (noalloc) {
    if (need > MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
    const mla_status st = scratch_for_current_device(&workspace);
    if (st != MLA_OK) return st;
    workspace_bytes = MLA_NOALLOC_SCRATCH_BYTES;
  }
  if (!workspace || !aligned16(workspace)) return MLA_ERR_WORKSPACE;
  if (workspace_bytes < need) return MLA_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  if (d_q == 128) {
    const PagedDecodeLayout L = paged_decode_layout(B, H, r, G);
    mla::DecodeAbsorbArgs aa{};
    aa.q = (const bf16*)q; aa.wuk = (const bf16*)w_uk; aa.qabs = (bf16*)(ws + L.d.qabs);
    aa.B = B; aa.H = H; aa.qscale = scale * mla::kLog2e;
    mla::DecodeSoloArgs sa{};
    sa.qabs = aa.qabs; sa.cache = (const bf16*)c_cache; sa.cu = cu_seqlens;
    sa.lens = (const int*)(ws + L.lens); sa.cu_t = (const int*)(ws + L.cu_t); sa.rt = (const int*)(ws + L.rt);
    sa.part_o = (bf16*)(ws + L.d.part_o); sa.part_ml = (float*)(ws + L.d.part_ml);
    sa.B = B; sa.H = H; sa.N = (int)total_len;
    mla::DecodeMergeArgs ma{};
    ma.part_o = sa.part_o; ma.part_ml = sa.part_ml;
    ma.wuv = (const bf16*)w_uv; ma.gate = (const bf16*)gate; ma.out = (bf16*)out;
    ma.B = B; ma.H = H; ma.G = G;
    launch_decode_solo<128, 128, 512, false>(aa, nullptr, cu_seqlens, (int)total_len, G, (int*)(ws + L.krange), sa, ma, s);
    return launch_status();
  }
  // every range must own at least one cache row (the merge relies on it)
  if ((long long)G > total_len) G = (int)total_len;
  const DecodeLayout L = decode_layout(B, H, r, G);

  mla::DecodeAbsorbArgs aa{};
  aa.q = (const bf16*)q; aa.wuk = (const bf16*)w_uk; aa.qabs = (bf16*)(ws + L.qabs);
  aa.B = B; aa.H = H; aa.qscale = scale * mla::kLog2e;
  mla::DecodeSplitArgs sa{};
  sa.qabs = aa.qabs; sa.cache = (const bf16*)c_cache; sa.cu = cu_seqlens;
  sa.part_o = (bf16*)(ws + L.part_o); sa.part_ml = (float*)(ws + L.part_ml);
  sa.B = B; sa.H = H; sa.G = G; sa.N = total_len;
  mla::DecodeMergeArgs ma{};
  ma.part_o = sa.part_o; ma.part_ml = sa.part_ml; ma.cu = cu_seqlens;
  ma.wuv = (const bf16*)w_uv; ma.gate = (const bf16*)gate; ma.out = (bf16*)out;
  ma.B = B; ma.H = H; ma.G = G; ma.N = total_len;
  if (d_q == 16) launch_decode_bf16<16, 16, 32>(aa, sa, ma, s);
  else launch_decode_bf16<64, 64, 256>(aa, sa, ma, s);
  return launch_status();
}

mla_status mla_absorb_decode(const void* q, const void* c_cache, const int32_t* cu_seqlens,
                             const void* w_uk, const void* w_uv, const void* gate, void* out,
                             int B, int H, int d_q, int d_v, int r, int64_t total_len, float scale,
                             int num_splits, mla_dtype dtype, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return decode_impl(q, c_cache, cu_seqlens, w_uk, w_uv, gate, out, B, H, d_q, d_v, r, total_len, scale,
                     num_splits, dtype, workspace, workspace_bytes, stream, false);
}

mla_status mla_absorb_decode_noalloc(const void* q, const void* c_cache, const int32_t* cu_seqlens,
                                     const void* w_uk, const void* w_uv, const void* gate, void* out,
                                     int B, int H, int d_q, int d_v, int r, int64_t total_len, float scale,
                                     int num_splits, mla_dtype dtype, void* stream) {
  return decode_impl(q, c_cache, cu_seqlens, w_uk, w_uv, gate, out, B, H, d_q, d_v, r, total_len, scale,
                     num_splits, dtype, nullptr, 0, stream, true);
}

size_t mla_absorb_decode_paged_workspace_size(int B, int H, int d_q, int r, int num_splits, mla_dtype dtype) {
  if (B <= 0 || H <= 0 || d_q <= 0 || r <= 0) return kBadSize;
  if (dtype != MLA_DTYPE_BF16) return kBadSize;
  const int G = num_splits > 0 ? num_splits : device_cu_count();
  if (G <= 0) return kBadSize;
  return paged_decode_layout(B, H, r, G).total;
}

mla_status mla_absorb_decode_paged(const void* q, const void* c_pages, const int32_t* block_table,
                                   const int32_t* seq_lens, const void* w_uk, const void* w_uv, const void* gate,
                                   void* out, int B, int H, int d_q, int d_v, int r, int64_t num_pages,
                                   int page_size, int max_pages, float scale, int num_splits, mla_dtype dtype,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !c_pages || !block_table || !seq_lens || !w_uk || !w_uv || !gate || !out) return MLA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || d_q <= 0 || d_v <= 0 || r <= 0) return MLA_ERR_INVALID_ARG;
  if (num_pages <= 0 || max_pages <= 0 || page_size < 32 || log2_exact(page_size) < 0) return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return MLA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, c_pages, block_table, seq_lens, w_uk, w_uv, gate, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MLA_ERR_INVALID_ARG;
  if (dtype != MLA_DTYPE_BF16) return dtype == MLA_DTYPE_F32 ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  if (!bf16_shape_supported(d_q, d_v, r) || H > 16 * mla::kDecodeWaves) return MLA_ERR_UNSUPPORTED;
  if (!paged_geometry_ok(B, r, num_pages, page_size, max_pages) || !fits(B, H, d_q > d_v ? d_q : d_v))
    return MLA_ERR_UNSUPPORTED;
  const int G = num_splits > 0 ? num_splits : device_cu_count();
  if (G <= 0) return MLA_ERR_HIP;
  const PagedDecodeLayout L = paged_decode_layout(B, H, r, G);
  if (!workspace || !aligned16(workspace)) return MLA_ERR_WORKSPACE;
  if (workspace_bytes < L.total) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;

  mla::DecodeAbsorbArgs aa{};
  aa.q = (const bf16*)q; aa.wuk = (const bf16*)w_uk; aa.qabs = (bf16*)(ws + L.d.qabs);
  aa.B = B; aa.H = H; aa.qscale = scale * mla::kLog2e;
  const int max_rows = max_pages * page_size;
  if (d_q == 128) {
    mla::DecodeSoloArgs sa{};
    sa.qabs = aa.qabs; sa.cache = (const bf16*)c_pages; sa.block_table = block_table;
    sa.lens = (const int*)(ws + L.lens); sa.cu_t = (const int*)(ws + L.cu_t); sa.rt = (const int*)(ws + L.rt);
    sa.part_o = (bf16*)(ws + L.d.part_o); sa.part_ml = (float*)(ws + L.d.part_ml);
    sa.B = B; sa.H = H;
    sa.page_shift = log2_exact(page_size); sa.max_pages = max_pages; sa.num_pages = (int)num_pages;
    mla::DecodeMergeArgs ma{};
    ma.part_o = sa.part_o; ma.part_ml = sa.part_ml;
    ma.wuv = (const bf16*)w_uv; ma.gate = (const bf16*)gate; ma.out = (bf16*)out;
    ma.B = B; ma.H = H; ma.G = G;
    launch_decode_solo<128, 128, 512, true>(aa, seq_lens, nullptr, max_rows, G, (int*)(ws + L.krange), sa, ma, s);
    return launch_status();
  }
  mla::DecodePagedArgs sa{};
  sa.qabs = aa.qabs; sa.pages = (const bf16*)c_pages; sa.block_table = block_table;
  sa.lens = (const int*)(ws + L.lens); sa.cu_t = (const int*)(ws + L.cu_t);
  sa.part_o = (bf16*)(ws + L.d.part_o); sa.part_ml = (float*)(ws + L.d.part_ml);
  sa.B = B; sa.H = H; sa.G = G;
  sa.page_shift = log2_exact(page_size); sa.max_pages = max_pages; sa.num_pages = (int)num_pages;
  mla::DecodeMergeArgs ma{};
  ma.part_o = sa.part_o; ma.part_ml = sa.part_ml; ma.cu = sa.cu_t; ma.n_dev = sa.cu_t + B;
  ma.wuv = (const bf16*)w_uv; ma.gate = (const bf16*)gate; ma.out = (bf16*)out;
  ma.B = B; ma.H = H; ma.G = G; ma.N = 0;
  if (d_q == 16) launch_decode_paged_bf16<16, 16, 32>(aa, seq_lens, max_rows, sa, ma, s);
  else launch_decode_paged_bf16<64, 64, 256>(aa, seq_lens, max_rows, sa, ma, s);
  return launch_status();
}

mla_status mla_cache_append_paged(const void* c_new, void* c_pages, const int32_t* block_table,
                                  const int32_t* positions, int B, int r, int64_t num_pages, int page_size,
                                  int max_pages, mla_dtype dtype, void* stream) {
  if (!c_new || !c_pages || !block_table || !positions) return MLA_ERR_INVALID_ARG;
  if (B <= 0 || r <= 0 || num_pages <= 0 || page_size <= 0 || max_pages <= 0) return MLA_ERR_INVALID_ARG;
  if (dtype != MLA_DTYPE_F32 && dtype != MLA_DTYPE_BF16) return MLA_ERR_INVALID_ARG;
  const void* ptrs[] = {c_new, c_pages, block_table, positions};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MLA_ERR_INVALID_ARG;
  const int row_bytes = r * (dtype == MLA_DTYPE_F32 ? 4 : 2);
  if (row_bytes % 16) return MLA_ERR_UNSUPPORTED;
  if (num_pages >= (1LL << 31) || (long long)max_pages * page_size >= (1LL << 31) || !fits(B, max_pages) ||
      !fits(num_pages, page_size, row_bytes) || B >= (1 << 30))
    return MLA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(mla::mla_cache_append_paged, dim3((B + 3) / 4), dim3(256), 0, (hipStream_t)stream,
                     (const char*)c_new, (char*)c_pages, block_table, positions, B, row_bytes, page_size, max_pages,
                     (int)num_pages);
  return launch_status();
}

size_t mla_absorb_prefill_backward_workspace_size(int B, int T, int H, int d_q, int d_v, int r, mla_dtype dtype) {
  if (B <= 0 || T <= 0 || H <= 0 || d_q <= 0 || d_v <= 0 || r <= 0) return kBadSize;
  if (dtype != MLA_DTYPE_BF16) return kBadSize;
  return backward_layout(B, T, H, d_q, d_v, r).total;
}

// The core backward; dgate rows are ldg elements apart (H d_v for the
// entry point, wider inside the layer backward's side-by-side gradients).
static mla_status prefill_backward_impl(const void* q, const void* c, const void* w_uk, const void* w_uv,
                                        const void* gate, const void* out, const float* lse, const void* dout,
                                        void* dq, void* dc, float* dw_uk, float* dw_uv, void* dgate, int ldg, int B,
                                        int T, int H, int d_q, int d_v, int r, float scale, mla_dtype dtype,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  const void* ptrs[] = {q, c, w_uk, w_uv, gate, out, lse, dout, dq, dc, dw_uk, dw_uv, dgate};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return MLA_ERR_INVALID_ARG;
  if (B <= 0 || T <= 0 || H <= 0 || d_q <= 0 || d_v <= 0 || r <= 0) return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return MLA_ERR_INVALID_ARG;
  if (dtype != MLA_DTYPE_BF16) return dtype == MLA_DTYPE_F32 ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  if (!bf16_shape_supported(d_q, d_v, r)) return MLA_ERR_UNSUPPORTED;
  // 32-bit offsets inside the weight-gradient GEMM descriptors
  const long long BT = (long long)B * T;
  if (BT >= (1LL << 31) || (long double)H * BT * r * 2 >= 2.0e9L || (long double)H * BT * d_q * 2 >= 2.0e9L ||
      (long double)H * BT * d_v * 2 >= 2.0e9L)
    return MLA_ERR_UNSUPPORTED;
  const BackwardLayout L = backward_layout(B, T, H, d_q, d_v, r);
  if (!workspace || !aligned16(workspace)) return MLA_ERR_WORKSPACE;
  if (workspace_bytes < L.total) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;

  mla::BwdPrepArgs pa{};
  pa.gate = (const bf16*)gate; pa.out = (const bf16*)out; pa.dout = (const bf16*)dout; pa.lse = lse;
  pa.dgate = (bf16*)dgate; pa.dov = (bf16*)(ws + L.dov); pa.ld = (float*)(ws + L.ld);
  pa.B = B; pa.T = T; pa.H = H; pa.DV = d_v; pa.ldg = ldg;
  bf16* wukT = (bf16*)(ws + L.wukT);
  bf16* wuvT = (bf16*)(ws + L.wuvT);
  launch_wuk_transpose((const bf16*)w_uk, wukT, H, d_q, r, s);
  launch_wuk_transpose((const bf16*)w_uv, wuvT, H, d_v, r, s);
  mla::BwdArgs ba{};
  ba.c = (const bf16*)c; ba.qabs = (bf16*)(ws + L.qabs); ba.dolat = (bf16*)(ws + L.dolat); ba.ld = pa.ld;
  ba.dov = pa.dov; ba.da = (bf16*)(ws + L.da); ba.dv = (bf16*)(ws + L.dv); ba.dc_part = (float*)(ws + L.part);
  ba.B = B; ba.T = T; ba.H = H; ba.scale = scale; ba.ntb = (T + 31) / 32; ba.nhg = L.nhg; ba.hpg = L.hpg;
  if (d_q == 16) launch_backward_bf16<16, 16, 32>(pa, ba, (const bf16*)q, wukT, wuvT, s);
  else if (d_q == 64) launch_backward_bf16<64, 64, 256>(pa, ba, (const bf16*)q, wukT, wuvT, s);
  else launch_backward_bf16<128, 128, 512>(pa, ba, (const bf16*)q, wukT, wuvT, s);

  // dc: sum of the head-group partials
  const long long n4 = BT * r / 4;
  hipLaunchKernelGGL(mla::mla_bwd_dc_sum, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, ba.dc_part,
                     (bf16*)dc, BT, r, L.nhg);
  // dq[:, h, :] = da[h] W_UK[h]^T
  launch_gemm_batched(ba.da, r, BT * r, (const bf16*)w_uk, r, (long long)d_q * r, (bf16*)dq, H * d_q, d_q, (int)BT, d_q,
                      r, 1.0f, H, s);
  // dW_UK[h] = q[:, h, :]^T da[h];  dW_UV[h] = dV[h]^T c
  const size_t q_bytes = (size_t)BT * H * d_q * 2, hr_bytes = (size_t)H * BT * r * 2,
               dv_bytes = (size_t)H * BT * d_v * 2, c_bytes = (size_t)BT * r * 2;
  launch_gemm_tn((const bf16*)q, q_bytes, H * d_q, d_q, ba.da, hr_bytes, r, BT * r, dw_uk, (long long)d_q * r, d_q,
                 r, (int)BT, H, s);
  launch_gemm_tn(ba.dv, dv_bytes, d_v, BT * d_v, (const bf16*)c, c_bytes, r, 0, dw_uv, (long long)d_v * r, d_v, r,
                 (int)BT, H, s);
  return launch_status();
}

mla_status mla_absorb_prefill_backward(const void* q, const void* c, const void* w_uk, const void* w_uv,
                                       const void* gate, const void* out, const float* lse, const void* dout,
                                       void* dq, void* dc, float* dw_uk, float* dw_uv, void* dgate, int B, int T,
                                       int H, int d_q, int d_v, int r, float scale, mla_dtype dtype, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return prefill_backward_impl(q, c, w_uk, w_uv, gate, out, lse, dout, dq, dc, dw_uk, dw_uv, dgate, H * d_v, B, T, H,
                               d_q, d_v, r, scale, dtype, workspace, workspace_bytes, stream);
}

// Shape checks shared by the full-layer forward, its training form and its backward.
static mla_status layer_shape_check(int B, int T, int D, int q_rank, int H, int d_q, int d_v, int r) {
  if (B <= 0 || T <= 0 || D <= 0 || q_rank <= 0 || H <= 0 || d_q <= 0 || d_v <= 0 || r <= 0)
    return MLA_ERR_INVALID_ARG;
  if (!bf16_shape_supported(d_q, d_v, r)) return MLA_ERR_UNSUPPORTED;
  // projection contractions come in 64-wide k tiles; normalised rows fit one wave
  if (D % 64 || q_rank % 64 || (H * d_v) % 64 || (H * d_q) % 8 || D % 8 || r % 8 || q_rank % 8)
    return MLA_ERR_UNSUPPORTED;
  if (r > 64 * 8 * mla::kNormMaxChunks || q_rank > 64 * 8 * mla::kNormMaxChunks) return MLA_ERR_UNSUPPORTED;
  if (!fits(B, T, D) || !fits(B, T, H, d_q > d_v ? d_q : d_v) || (long long)B * T >= (1LL << 31))
    return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

size_t mla_gated_forward_workspace_size(int B, int T, int q_rank, int H, int d_q, int d_v, int r,
                                        mla_dtype dtype) {
  if (B <= 0 || T <= 0 || q_rank <= 0 || H <= 0 || d_q <= 0 || d_v <= 0 || r <= 0) return kBadSize;
  if (dtype != MLA_DTYPE_BF16) return kBadSize;
  return forward_layout(B, T, q_rank, H, d_q, d_v, r).total;
}

mla_status mla_gated_forward(const void* x, const void* w_kv_down, const void* kv_norm, const void* w_q_down,
                             const void* q_norm, const void* w_q_up, const void* w_uk, const void* w_uv,
                             const void* w_gate, const void* w_o, void* y, int B, int T, int D, int q_rank,
                             int H, int d_q, int d_v, int r, float eps, float scale, mla_dtype dtype,
                             void* workspace, size_t workspace_bytes, void* stream) {
  const void* ptrs[] = {x, w_kv_down, kv_norm, w_q_down, q_norm, w_q_up, w_uk, w_uv, w_gate, w_o, y};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return MLA_ERR_INVALID_ARG;
  if (B <= 0 || T <= 0 || D <= 0 || q_rank <= 0 || H <= 0 || d_q <= 0 || d_v <= 0 || r <= 0)
    return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !std::isfinite(eps) || eps < 0.0f) return MLA_ERR_INVALID_ARG;
  if (dtype != MLA_DTYPE_BF16) return MLA_ERR_UNSUPPORTED;
  const mla_status st0 = layer_shape_check(B, T, D, q_rank, H, d_q, d_v, r);
  if (st0 != MLA_OK) return st0;
  const ForwardLayout L = forward_layout(B, T, q_rank, H, d_q, d_v, r);
  if (!workspace || !aligned16(workspace)) return MLA_ERR_WORKSPACE;
  if (workspace_bytes < L.total) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int N = B * T;
  const bf16* xb = (const bf16*)x;
  bf16* c = (bf16*)(ws + L.c);
  bf16* ql = (bf16*)(ws + L.ql);
  bf16* q = (bf16*)(ws + L.q);
  bf16* gate = (bf16*)(ws + L.gate);
  bf16* o = (bf16*)(ws + L.o);
  // latent: c = RMSNorm(W_down x)
  launch_gemm(xb, (const bf16*)w_kv_down, c, N, r, D, s);
  launch_rmsnorm(c, c, (const bf16*)kv_norm, nullptr, N, r, eps, s);
  // query low-rank path: q = W_q_up RMSNorm(W_q_down x)
  launch_gemm(xb, (const bf16*)w_q_down, ql, N, q_rank, D, s);
  launch_rmsnorm(ql, ql, (const bf16*)q_norm, nullptr, N, q_rank, eps, s);
  launch_gemm(ql, (const bf16*)w_q_up, q, N, H * d_q, q_rank, s);
  // gate pre-activations
  launch_gemm(xb, (const bf16*)w_gate, gate, N, H * d_v, D, s);
  // absorbed core: gated head outputs, flattened head-major
  const mla_status st = mla_absorb_prefill(q, c, w_uk, w_uv, gate, o, B, T, H, d_q, d_v, r, scale, dtype,
                                           ws + L.core, L.total - L.core, stream);
  if (st != MLA_OK) return st;
  // output projection
  launch_gemm(o, (const bf16*)w_o, (bf16*)y, N, D, H * d_v, s);
  return launch_status();
}


size_t mla_gated_train_state_size(int B, int T, int q_rank, int H, int d_q, int d_v, int r, mla_dtype dtype) {
  if (B <= 0 || T <= 0 || q_rank <= 0 || H <= 0 || d_q <= 0 || d_v <= 0 || r <= 0) return kBadSize;
  if (dtype != MLA_DTYPE_BF16) return kBadSize;
  return train_layout(B, T, q_rank, H, d_q, d_v, r).total;
}

mla_status mla_gated_forward_train(const void* x, const void* w_kv_down, const void* kv_norm, const void* w_q_down,
                                   const void* q_norm, const void* w_q_up, const void* w_uk, const void* w_uv,
                                   const void* w_gate, const void* w_o, void* y, int B, int T, int D, int q_rank,
                                   int H, int d_q, int d_v, int r, float eps, float scale, mla_dtype dtype,
                                   void* state, size_t state_bytes, void* stream) {
  const void* ptrs[] = {x, w_kv_down, kv_norm, w_q_down, q_norm, w_q_up, w_uk, w_uv, w_gate, w_o, y};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !std::isfinite(eps) || eps < 0.0f) return MLA_ERR_INVALID_ARG;
  if (dtype != MLA_DTYPE_BF16) return dtype == MLA_DTYPE_F32 ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  const mla_status st0 = layer_shape_check(B, T, D, q_rank, H, d_q, d_v, r);
  if (st0 != MLA_OK) return st0;
  if (!fits(B, H, T)) return MLA_ERR_UNSUPPORTED;
  const TrainLayout L = train_layout(B, T, q_rank, H, d_q, d_v, r);
  if (!state || !aligned16(state)) return MLA_ERR_WORKSPACE;
  if (state_bytes < L.total) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* st = (char*)state;
  const int N = B * T;
  const bf16* xb = (const bf16*)x;
  bf16* c_pre = (bf16*)(st + L.c_pre);
  bf16* c = (bf16*)(st + L.c);
  bf16* ql_pre = (bf16*)(st + L.ql_pre);
  bf16* ql = (bf16*)(st + L.ql);
  bf16* q = (bf16*)(st + L.q);
  bf16* gate = (bf16*)(st + L.gate);
  bf16* o = (bf16*)(st + L.o);
  launch_gemm(xb, (const bf16*)w_kv_down, c_pre, N, r, D, s);
  launch_rmsnorm(c_pre, c, (const bf16*)kv_norm, (float*)(st + L.rstd_c), N, r, eps, s);
  launch_gemm(xb, (const bf16*)w_q_down, ql_pre, N, q_rank, D, s);
  launch_rmsnorm(ql_pre, ql, (const bf16*)q_norm, (float*)(st + L.rstd_q), N, q_rank, eps, s);
  launch_gemm(ql, (const bf16*)w_q_up, q, N, H * d_q, q_rank, s);
  launch_gemm(xb, (const bf16*)w_gate, gate, N, H * d_v, D, s);
  const mla_status st1 = mla_absorb_prefill_train(q, c, w_uk, w_uv, gate, o, (float*)(st + L.lse), B, T, H, d_q,
                                                  d_v, r, scale, dtype, st + L.core, L.total - L.core, stream);
  if (st1 != MLA_OK) return st1;
  launch_gemm(o, (const bf16*)w_o, (bf16*)y, N, D, H * d_v, s);
  return launch_status();
}

size_t mla_gated_backward_workspace_size(int B, int T, int D, int q_rank, int H, int d_q, int d_v, int r,
                                         mla_dtype dtype) {
  if (B <= 0 || T <= 0 || D <= 0 || q_rank <= 0 || H <= 0 || d_q <= 0 || d_v <= 0 || r <= 0) return kBadSize;
  if (dtype != MLA_DTYPE_BF16) return kBadSize;
  return layer_bwd_layout(B, T, D, q_rank, H, d_q, d_v, r).total;
}

mla_status mla_gated_backward(const void* x, const void* w_kv_down, const void* kv_norm, const void* w_q_down,
                              const void* q_norm, const void* w_q_up, const void* w_uk, const void* w_uv,
                              const void* w_gate, const void* w_o, const void* dy, const void* state,
                              size_t state_bytes, void* dx, float* dw_kv_down, float* dkv_norm, float* dw_q_down,
                              float* dq_norm, float* dw_q_up, float* dw_uk, float* dw_uv, float* dw_gate,
                              float* dw_o, int B, int T, int D, int q_rank, int H, int d_q, int d_v, int r,
                              float scale, mla_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  const void* ptrs[] = {x, w_kv_down, kv_norm, w_q_down, q_norm, w_q_up, w_uk, w_uv, w_gate, w_o, dy, dx,
                        dw_kv_down, dkv_norm, dw_q_down, dq_norm, dw_q_up, dw_uk, dw_uv, dw_gate, dw_o};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return MLA_ERR_INVALID_ARG;
  if (dtype != MLA_DTYPE_BF16) return dtype == MLA_DTYPE_F32 ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  const mla_status st0 = layer_shape_check(B, T, D, q_rank, H, d_q, d_v, r);
  if (st0 != MLA_OK) return st0;
  const long long N = (long long)B * T;
  const int HQ = H * d_q, HV = H * d_v;
  const LayerBwdLayout L = layer_bwd_layout(B, T, D, q_rank, H, d_q, d_v, r);
  // the weight-gradient products address each token-major operand with 32-bit offsets
  if ((long double)N * L.Kc * 2 >= 2.0e9L || (long double)N * D * 2 >= 2.0e9L || (long double)N * HQ * 2 >= 2.0e9L ||
      (long double)N * HV * 2 >= 2.0e9L)
    return MLA_ERR_UNSUPPORTED;
  const TrainLayout TL = train_layout(B, T, q_rank, H, d_q, d_v, r);
  if (!state || !aligned16(state) || state_bytes < TL.total) return MLA_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace)) return MLA_ERR_WORKSPACE;
  if (workspace_bytes < L.total) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const char* st = (const char*)state;
  char* ws = (char*)workspace;
  const bf16* xb = (const bf16*)x;
  const bf16* dyb = (const bf16*)dy;
  const bf16* o = (const bf16*)(st + TL.o);
  bf16* gcat = (bf16*)(ws + L.gcat);
  bf16* dout = (bf16*)(ws + L.dout);
  bf16* dqb = (bf16*)(ws + L.dq);
  bf16* dcb = (bf16*)(ws + L.dc);
  bf16* dql = (bf16*)(ws + L.dql);
  bf16* woT = (bf16*)(ws + L.woT);
  bf16* wqupT = (bf16*)(ws + L.wqupT);
  bf16* wcatT = (bf16*)(ws + L.wcatT);
  float* part = (float*)(ws + L.part);
  const int Kc = L.Kc;

  // output projection y = o W_o^T: dout = dy W_o, dW_o = dy^T o
  launch_transpose_into((const bf16*)w_o, D, HV, woT, D, s);
  launch_gemm(dyb, woT, dout, (int)N, HV, D, s);
  launch_gemm_tn(dyb, (size_t)N * D * 2, D, 0, o, (size_t)N * HV * 2, HV, 0, dw_o, 0, D, HV, (int)N, 1, s);
  // the core: dq, dc, dW_UK, dW_UV and the gate gradient into gcat[:, 0:HV]
  const mla_status st1 = prefill_backward_impl(st + TL.q, st + TL.c, w_uk, w_uv, st + TL.gate, o,
                                               (const float*)(st + TL.lse), dout, dqb, dcb, dw_uk, dw_uv, gcat, Kc, B,
                                               T, H, d_q, d_v, r, scale, dtype, ws + L.core, L.total - L.core, stream);
  if (st1 != MLA_OK) return st1;
  // query up-projection q = ql W_q_up^T: dql = dq W_q_up, dW_q_up = dq^T ql
  launch_transpose_into((const bf16*)w_q_up, HQ, q_rank, wqupT, HQ, s);
  launch_gemm(dqb, wqupT, dql, (int)N, q_rank, HQ, s);
  launch_gemm_tn(dqb, (size_t)N * HQ * 2, HQ, 0, (const bf16*)(st + TL.ql), (size_t)N * q_rank * 2, q_rank, 0, dw_q_up,
                 0, HQ, q_rank, (int)N, 1, s);
  // the two norms: gradients of their inputs into gcat, gain gradients
  launch_rmsnorm_backward(dql, q_rank, (const bf16*)(st + TL.ql_pre), (const float*)(st + TL.rstd_q),
                          (const bf16*)q_norm, gcat + HV, Kc, part, dq_norm, (int)N, q_rank, s);
  launch_rmsnorm_backward(dcb, r, (const bf16*)(st + TL.c_pre), (const float*)(st + TL.rstd_c), (const bf16*)kv_norm,
                          gcat + HV + q_rank, Kc, part, dkv_norm, (int)N, r, s);
  // the three products of x: dx = gcat [W_gate; W_q_down; W_kv_down], and their weight gradients
  launch_transpose_into((const bf16*)w_gate, HV, D, wcatT, Kc, s);
  launch_transpose_into((const bf16*)w_q_down, q_rank, D, wcatT + HV, Kc, s);
  launch_transpose_into((const bf16*)w_kv_down, r, D, wcatT + HV + q_rank, Kc, s);
  launch_gemm_batched(gcat, Kc, 0, wcatT, Kc, 0, (bf16*)dx, D, 0, (int)N, D, Kc, 1.0f, 1, s);
  const size_t gcat_bytes = (size_t)N * Kc * 2, x_bytes = (size_t)N * D * 2;
  launch_gemm_tn(gcat, gcat_bytes, Kc, 0, xb, x_bytes, D, 0, dw_gate, 0, HV, D, (int)N, 1, s);
  launch_gemm_tn(gcat + HV, gcat_bytes - (size_t)HV * 2, Kc, 0, xb, x_bytes, D, 0, dw_q_down, 0, q_rank, D, (int)N, 1,
                 s);
  launch_gemm_tn(gcat + HV + q_rank, gcat_bytes - (size_t)(HV + q_rank) * 2, Kc, 0, xb, x_bytes, D, 0, dw_kv_down, 0,
                 r, D, (int)N, 1, s);
  return launch_status();
}

}  // extern "C"
