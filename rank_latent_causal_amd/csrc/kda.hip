// Host side of chunk_kda: argument checks, workspace layout and the two
// launches behind kda.h.
#include "kda.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kda_bf16.h"

namespace {

constexpr size_t kBad = (size_t)-1;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool widths_supported(int K, int V) { return K == V && (K == 16 || K == 64 || K == 128); }

size_t slot_bytes(int K) {
  switch (K) {
    case 16: return kda::KdaDims<16, 16>::SLOT;
    case 64: return kda::KdaDims<64, 64>::SLOT;
    default: return kda::KdaDims<128, 128>::SLOT;
  }
}

template <int DK, int DV, int VB>
void launch(kda::KdaArgs a, hipStream_t s) {
  const long long slots = (long long)a.B * a.HV * a.NC;
  hipLaunchKernelGGL((kda::kda_intra<DK, DV>), dim3((unsigned)slots), dim3(64 * kda::intra_waves<DK>()), 0, s, a);
  constexpr int NVB = DV / VB;
  const long long heads = (long long)a.B * a.HV;
  a.xcd_map = (NVB > 1 && heads % 8 == 0) ? 1 : 0;
  // two waves per SIMD where the value tiles of a block split evenly
  constexpr int NW = (VB / 16) % 2 == 0 ? 8 : 4;
  hipLaunchKernelGGL((kda::kda_state<DK, DV, VB, NW>), dim3((unsigned)(heads * NVB)), dim3(64 * NW), 0, s, a);
}

}  // namespace

extern "C" {

size_t kda_chunk_workspace_size(int B, int T, int H, int G, int K, int V, mla_dtype dtype) {
  if (B <= 0 || T <= 0 || H <= 0 || G <= 0 || K <= 0 || V <= 0) return kBad;
  if (dtype != MLA_DTYPE_BF16 || !widths_supported(K, V)) return kBad;
  const long double n = (long double)B * G * H * ((T + kda::kC - 1) / kda::kC) * slot_bytes(K);
  if (n >= 1.0e18L) return kBad;
  return (size_t)n;
}

mla_status kda_chunk_forward(const void* q, const void* k, const void* v, const float* g, const float* beta,
                             const float* initial_state, void* o, float* final_state, int B, int T, int H, int G,
                             int K, int V, mla_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  const void* req[] = {q, k, v, g, beta, o};
  for (const void* p : req)
    if (!p || !aligned16(p)) return MLA_ERR_INVALID_ARG;
  if ((initial_state && !aligned16(initial_state)) || (final_state && !aligned16(final_state)))
    return MLA_ERR_INVALID_ARG;
  if (B <= 0 || T <= 0 || H <= 0 || G <= 0 || K <= 0 || V <= 0) return MLA_ERR_INVALID_ARG;
  if (dtype != MLA_DTYPE_BF16) return dtype == MLA_DTYPE_F32 ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  if (!widths_supported(K, V)) return MLA_ERR_UNSUPPORTED;
  // grid and element offsets: every index below stays far inside int32 / int64
  const long long HV = (long long)G * H, NC = (T + kda::kC - 1) / kda::kC;
  if (HV >= (1LL << 20) || (long double)B * HV * NC >= 2.0e9L || (long double)B * T * HV * (K > V ? K : V) >= 4.0e18L)
    return MLA_ERR_UNSUPPORTED;
  // the in-chunk kernel copies q, k and g with 32-bit offsets inside one batch
  if ((long double)T * H * K * 2 >= 2.0e9L || (long double)T * HV * K * 4 >= 2.0e9L) return MLA_ERR_UNSUPPORTED;
  const size_t need = kda_chunk_workspace_size(B, T, H, G, K, V, dtype);
  if (need == kBad) return MLA_ERR_UNSUPPORTED;
  if (!workspace || !aligned16(workspace)) return MLA_ERR_WORKSPACE;
  if (workspace_bytes < need) return MLA_ERR_WORKSPACE;

  kda::KdaArgs a{};
  a.q = (const mla::bf16*)q; a.k = (const mla::bf16*)k; a.v = (const mla::bf16*)v;
  a.g = g; a.beta = beta; a.s0 = initial_state; a.o = (mla::bf16*)o; a.s_out = final_state;
  a.ws = (char*)workspace;
  a.B = B; a.T = T; a.H = H; a.G = G; a.HV = (int)HV; a.NC = (int)NC;
  hipStream_t s = (hipStream_t)stream;
  if (K == 16) launch<16, 16, 16>(a, s);
  else if (K == 64) launch<64, 64, 32>(a, s);
  else launch<128, 128, 64>(a, s);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
