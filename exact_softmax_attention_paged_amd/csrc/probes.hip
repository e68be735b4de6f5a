// Device-ceiling probes for gfx950 (libattn_probes.so): an HBM read stream with 16-byte loads,
// a back-to-back v_mfma_f32_32x32x16_bf16 loop with a shader-clock reading, and an LDS read
// loop in the two read forms of the prefill kernel (ds_read_b128, ds_read_b64_tr_b16). See
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

constexpr int kLdsWaves = 8;
constexpr int kLdsBytes = 64 * 1024;
constexpr int kLdsBatch = 8;           // independent reads per wave and round

typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// The 64 KiB tile is filled once, then every wave reads it in rounds of kLdsBatch independent
// reads at addresses that move with the round (so no read is loop-invariant), folding what it
// reads into one word. TR = false: ds_read_b128, lane l at 16 l within a 1 KiB row. TR = true:
// ds_read_b64_tr_b16 with the prefill kernel's V^T addressing for head_size 128 (rows
// 4 (l / 32) + (l % 16) / 4 of a 256-byte-row tile, 16-byte chunks XOR-swizzled per row).
template <bool TR>
__global__ __launch_bounds__(kLdsWaves * 64) void lds_read_kernel(uint64_t* clocks, uint32_t* sink,
                                                                  int32_t iters) {
  __shared__ __attribute__((aligned(1024))) unsigned char tile[kLdsBytes];
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  for (int i = threadIdx.x; i < kLdsBytes / 4; i += kLdsWaves * 64)
    reinterpret_cast<uint32_t*>(tile)[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  uint32_t lane_off;
  if (TR) {
    const int rr = 4 * (lane / 32) + (lane % 16) / 4;
    const int ch = 2 * ((lane / 16) % 2) + (lane % 4) / 2;
    const int swz = ((rr & 3) << 2) | ((rr >> 2) & 3);
    lane_off = (uint32_t)(rr * 256 + 16 * (ch ^ swz) + 8 * (lane % 2));
  } else {
    lane_off = (uint32_t)(16 * lane);
  }
  const uint32_t base = (uint32_t)(uintptr_t)tile + lane_off;
  uint32_t acc = 0;
  uint64_t t0 = 0, r0 = 0;
  if (wave == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
    // a round's reads: 8 KiB apart (b128) or 4 KiB apart (transposing reads cover 16 rows of
    // 256 bytes), shifted by the wave and the round, always inside the tile
    const uint32_t shift = (uint32_t)(((it + wave) % 8) * 1024);
    asm volatile("" ::: "memory");       // no read may be moved out of its round
    if (TR) {
      shortx4 v[kLdsBatch];
#pragma unroll
      for (int k = 0; k < kLdsBatch; ++k)
        v[k] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_shortx4*)(uintptr_t)(base + ((shift + k * 4096u) & (kLdsBytes - 1))));
#pragma unroll
      for (int k = 0; k < kLdsBatch; ++k)
        acc ^= (uint32_t)(uint16_t)v[k][0] ^ ((uint32_t)(uint16_t)v[k][3] << 16);
    } else {
      u32x4 v[kLdsBatch];
#pragma unroll
      for (int k = 0; k < kLdsBatch; ++k)
        v[k] = *(const lds_u32x4*)(uintptr_t)(base + ((shift + k * 8192u) & (kLdsBytes - 1)));
#pragma unroll
      for (int k = 0; k < kLdsBatch; ++k) acc ^= v[k][0] ^ v[k][3];
    }
  }
  sink[(uint64_t)blockIdx.x * kLdsWaves * 64 + threadIdx.x] = acc;
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

int32_t attn_probe_lds_read(uint64_t* clocks, uint32_t* sink, int32_t workgroups, int32_t iters,
                            int32_t transposing, void* stream) {
  if (clocks == nullptr || sink == nullptr || workgroups <= 0 || iters <= 0) return 1;
  if (transposing)
    hipLaunchKernelGGL(lds_read_kernel<true>, dim3(workgroups), dim3(kLdsWaves * 64), 0,
                       static_cast<hipStream_t>(stream), clocks, sink, iters);
  else
    hipLaunchKernelGGL(lds_read_kernel<false>, dim3(workgroups), dim3(kLdsWaves * 64), 0,
                       static_cast<hipStream_t>(stream), clocks, sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
