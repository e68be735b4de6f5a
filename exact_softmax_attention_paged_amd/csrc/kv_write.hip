// KV-cache write through slot_mapping, for gfx950.
//
// The new tokens' K and V rows are stored in the paged cache at the flat slots the batch
// metadata gives ("[vLLM] FlashAttention" page: slot_mapping beside block_table in the
// FlashAttentionMetadata section; block_table and slot_mapping give direct access to a
// non-contiguous cache, "왜 이 설계인가" item 2; cache shape from the FlashAttentionBackend
// section). Slot s is block s / block_size, offset s % block_size, the same split the block
// table uses for reads. Negative slots (padding tokens) and slots past the cache are skipped,
// so a bad slot can never write outside the cache.
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

}  // namespace

hipError_t launch_kv_write(const KvWriteParams& p, hipStream_t stream) {
  const int64_t total = p.num_tokens * 2 * p.row_chunks;
  if (total <= 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
