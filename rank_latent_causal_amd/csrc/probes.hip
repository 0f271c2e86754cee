// Measurement probes for bench.py (a library of their own, not part of the
// MLA / KDA C ABI): the sustained bf16 MFMA rate and the sustained HBM read
// rate of the device they run on, the measured peaks the benchmark states
// its roofline fractions against next to the published ones.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

typedef __bf16 pbf16x8 __attribute__((ext_vector_type(8)));
typedef float pf32x4 __attribute__((ext_vector_type(4)));

// 8 waves per workgroup, one workgroup per CU: each wave runs 4 independent
// chains of 16x16x32 bf16 MFMAs on operands held in registers (random values
// from `src`, so the rate is the one real data sees).
__global__ void __launch_bounds__(512) probe_mfma_kernel(const pbf16x8* __restrict__ src, float* __restrict__ sink,
                                                         int iters) {
  const int t = blockIdx.x * 512 + threadIdx.x;
  const pbf16x8 a0 = src[(t * 4 + 0) & 4095], a1 = src[(t * 4 + 1) & 4095];
  const pbf16x8 b0 = src[(t * 4 + 2) & 4095], b1 = src[(t * 4 + 3) & 4095];
  pf32x4 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b0, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b1, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, c3, 0, 0, 0);
    }
  }
  const pf32x4 s = c0 + c1 + c2 + c3;
  sink[t] = s[0] + s[1] + s[2] + s[3];
}

// Grid-stride 16-byte reads, four in flight per thread; the XOR of what was
// read is stored only if it equals an arbitrary constant, which keeps the
// loads without writing anything in practice.
__global__ void __launch_bounds__(256) probe_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                         unsigned* __restrict__ sink) {
  unsigned acc = 0;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
    acc ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w ^ v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^
           v3.w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

extern "C" {

// One launch of the MFMA loop over `blocks` workgroups (flops per launch:
// blocks * 8 waves * iters * 32 MFMAs * 16384).  src: 4096 x 16 bytes of
// bf16 operands; sink: blocks * 512 floats.  Returns hipError_t as int.
int probe_mfma_bf16(const void* src, float* sink, int blocks, int iters, void* stream) {
  if (!src || !sink || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream, (const pbf16x8*)src, sink,
                     iters);
  return (int)hipGetLastError();
}

// One streaming read of `bytes` (a multiple of 16) from src; sink holds
// `blocks` unsigned values.
int probe_stream_read(const void* src, size_t bytes, unsigned* sink, int blocks, void* stream) {
  if (!src || !sink || blocks <= 0 || bytes % 16) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint4*)src,
                     bytes / 16, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
