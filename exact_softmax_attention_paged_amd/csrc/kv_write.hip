// KV-cache write through slot_mapping, for gfx950.
//
// The new tokens' K and V rows are stored in the paged cache at the flat slots the batch
// metadata gives ("[vLLM] FlashAttention" page: slot_mapping beside block_table in the
// FlashAttentionMetadata section; block_table and slot_mapping give direct access to a
// non-contiguous cache, "왜 이 설계인가" item 2; cache shape from the FlashAttentionBackend
// section). Slot s is block s / block_size, offset s % block_size, the same split the block
// table uses for reads. Negative slots (padding tokens) and slots past the cache are skipped,
// so a bad slot can never write outside the cache. An E4M3 cache (per-tensor scales, bf16
// input) is written by a second kernel that quantises on the way.
//
// Pure data movement, HBM bound: each thread moves one 16-byte chunk of one token's K or V
// row (a token's rows of all kv heads are contiguous in the cache). Consecutive threads take
// consecutive chunks, so both the loads (rows of key/value with any 16-byte-aligned stride)
// and the stores (one contiguous run per token and half) are fully coalesced.
#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

__global__ __launch_bounds__(256) void kv_write_kernel(const KvWriteParams p) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;      // global chunk index
  const int64_t per_half = p.row_chunks;                          // 16-byte chunks per row
  const int64_t per_token = 2 * per_half;
  const int64_t t = g / per_token;
  if (t >= p.num_tokens) return;
  const int64_t c = g - t * per_token;
  const bool is_v = c >= per_half;
  const int64_t chunk = is_v ? c - per_half : c;
  const int64_t slot = p.slot_mapping[t];
  if (slot < 0 || slot >= p.num_slots) return;                    // padding or out of range
  const unsigned char* src = static_cast<const unsigned char*>(is_v ? p.value : p.key) +
                             t * (is_v ? p.value_stride_bytes : p.key_stride_bytes);
  unsigned char* dst = static_cast<unsigned char*>(p.kv_cache) +
                       (is_v ? p.v_offset_bytes : 0) + slot * p.slot_bytes;
  const u32x4 v = *reinterpret_cast<const u32x4*>(src + chunk * 16);
  *reinterpret_cast<u32x4*>(dst + chunk * 16) = v;
}

// E4M3 cache: each thread turns 16 bf16 inputs (32 bytes) into 16 codes (16 bytes). The code of
// x is the E4M3 value nearest to x / scale (fp32 quotient, ties to even, v_cvt_pk_fp8_f32),
// with magnitudes beyond 448 saturated first (the instruction alone would give NaN there).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float e4m3_saturate(float y) {
  return fabsf(y) > 448.f ? copysignf(448.f, y) : y;   // NaN passes through
}

__global__ __launch_bounds__(256) void kv_write_fp8_kernel(const KvWriteParams p) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_half = p.row_chunks;                          // 16-code chunks per row
  const int64_t per_token = 2 * per_half;
  const int64_t t = g / per_token;
  if (t >= p.num_tokens) return;
  const int64_t c = g - t * per_token;
  const bool is_v = c >= per_half;
  const int64_t chunk = is_v ? c - per_half : c;
  const int64_t slot = p.slot_mapping[t];
  if (slot < 0 || slot >= p.num_slots) return;                    // padding or out of range
  const unsigned char* src = static_cast<const unsigned char*>(is_v ? p.value : p.key) +
                             t * (is_v ? p.value_stride_bytes : p.key_stride_bytes) + chunk * 32;
  const float scale = is_v ? p.v_scale : p.k_scale;
  const u32x4 a = *reinterpret_cast<const u32x4*>(src);
  const u32x4 b = *reinterpret_cast<const u32x4*>(src + 16);
  const uint32_t in[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};   // 2 bf16 each
  u32x4 out;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t x0 = in[2 * w], x1 = in[2 * w + 1];
    const float f0 = e4m3_saturate(bf16_bits_to_f32(x0 & 0xFFFFu) / scale);
    const float f1 = e4m3_saturate(bf16_bits_to_f32(x0 >> 16) / scale);
    const float f2 = e4m3_saturate(bf16_bits_to_f32(x1 & 0xFFFFu) / scale);
    const float f3 = e4m3_saturate(bf16_bits_to_f32(x1 >> 16) / scale);
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, word, true);
    out[w] = (uint32_t)word;
  }
  unsigned char* dst = static_cast<unsigned char*>(p.kv_cache) +
                       (is_v ? p.v_offset_bytes : 0) + slot * p.slot_bytes + chunk * 16;
  *reinterpret_cast<u32x4*>(dst) = out;
}

}  // namespace

hipError_t launch_kv_write_fp8(const KvWriteParams& p, hipStream_t stream) {
  const int64_t total = p.num_tokens * 2 * p.row_chunks;
  if (total <= 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(kv_write_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_kv_write(const KvWriteParams& p, hipStream_t stream) {
  const int64_t total = p.num_tokens * 2 * p.row_chunks;
  if (total <= 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
