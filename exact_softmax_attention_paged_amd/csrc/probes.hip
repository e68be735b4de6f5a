// Device-ceiling probes for gfx950 (libattn_probes.so): an HBM read stream with 16-byte loads
// and a back-to-back v_mfma_f32_32x32x16_bf16 loop with a shader-clock reading. See
// include/attn_probes.h. Measurement only: nothing here is part of the attention path.
#include "attn_probes.h"

#include <hip/hip_runtime.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;

template <bool NT>
__global__ __launch_bounds__(kReadThreads) void read_stream_kernel(const u32x4* __restrict__ src,
                                                                   uint64_t n, uint32_t* sink) {
  uint32_t acc = 0;
  const uint64_t stride = (uint64_t)gridDim.x * kReadThreads * kReadUnroll;
  for (uint64_t base = (uint64_t)blockIdx.x * kReadThreads * kReadUnroll + threadIdx.x; base < n;
       base += stride) {
    // n is a multiple of kReadThreads * kReadUnroll, so a chunk that starts below n is whole
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const u32x4* a = src + base + (uint64_t)u * kReadThreads;
      v[u] = NT ? __builtin_nontemporal_load(a) : *a;
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  sink[(uint64_t)blockIdx.x * kReadThreads + threadIdx.x] = acc;
}

constexpr int kMfmaWaves = 8;
constexpr int kChains = 4;

__global__ __launch_bounds__(kMfmaWaves * 64) void mfma_loop_kernel(uint64_t* clocks, float* sink,
                                                                    int32_t iters) {
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  // operands: small exact bf16 values that differ per lane (no denormals, no overflow)
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.125f * (float)((lane + e) % 8) - 0.5f);
    b[e] = (__bf16)(0.0625f * (float)((lane * 3 + e) % 8) - 0.25f);
  }
  floatx16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  uint64_t t0 = 0, r0 = 0;
  if (wave == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  if (lane == 0) sink[(uint64_t)blockIdx.x * kMfmaWaves + wave] = s;
  if (wave == 0) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) {
      uint64_t* c = clocks + 4 * (uint64_t)blockIdx.x;
      c[0] = t0;
      c[1] = t1;
      c[2] = r0;
      c[3] = r1;
    }
  }
}

}  // namespace

extern "C" {

int32_t attn_probe_read_stream(const void* src, uint64_t bytes, uint32_t* sink,
                               int32_t workgroups, int32_t nontemporal, void* stream) {
  if (src == nullptr || sink == nullptr || bytes == 0 ||
      bytes % (16 * kReadThreads * kReadUnroll) != 0 ||
      (uintptr_t)src % 16 != 0 || workgroups <= 0)
    return 1;
  if (nontemporal)
    hipLaunchKernelGGL(read_stream_kernel<true>, dim3(workgroups), dim3(kReadThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                       bytes / 16, sink);
  else
    hipLaunchKernelGGL(read_stream_kernel<false>, dim3(workgroups), dim3(kReadThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                       bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int32_t attn_probe_mfma_loop(uint64_t* clocks, float* sink, int32_t workgroups, int32_t iters,
                             void* stream) {
  if (clocks == nullptr || sink == nullptr || workgroups <= 0 || iters <= 0) return 1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(workgroups), dim3(kMfmaWaves * 64), 0,
                     static_cast<hipStream_t>(stream), clocks, sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
