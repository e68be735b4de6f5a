// C-ABI layer of libattn.so: argument validation, workspace sizing, the decode/prefill
// dispatch from host scalars, and the launches on the caller's stream. See include/attn.h.
#include "attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "kernels.hpp"

namespace {

// Device memory of attn_varlen_fwd_noalloc: the split-KV partial results and the decode
// schedule, in a fixed array that every GPU the library runs on holds until the process ends.
// Host code never passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol): its device address is looked up once per device with hipGetSymbolAddress, and
// that address is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call there).
attn_status scratch_address(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return ATTN_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return ATTN_OK;
}

// Split-KV partition length when the descriptor leaves it at 0: the longest of 16384, 8192,
// ..., 256 keys that still gives the split kernel at least 2048 workgroups (counted from
// max_seq_len, i.e. an upper bound), else 256. With the longest-first decode schedule, longer
// partitions measured faster on gfx950 as long as the grid keeps about four workgroups per
// CU slot (two per CU): fewer workgroup prologues and partial results, and no merge pass for
// requests that fit one partition (paged GQA decode, 256 requests of 512..8192 keys, 32 q / 8
// kv heads: 0.843 / 0.836 / 0.821 ms with 2048 / 4096 / 8192 keys; 120 requests of 4K..32K
// keys, 64 q / 8 kv heads: 1.537 / 1.523 / 1.503 ms with 2048 / 4096 / 8192 and 1.516 ms
// with 16384, where the grid drops to 1920 workgroups).
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int32_t partition_tokens(const attn_desc* d) {
  if (d->partition_tokens > 0) return d->partition_tokens;
  const int64_t per_part = (int64_t)d->num_decodes * d->num_kv_heads *
                           ceil_div(d->num_heads / d->num_kv_heads, 16);
  for (int32_t P = attn::kMaxPartitionTokens; P > 256; P /= 2)
    if (per_part * ceil_div(d->max_seq_len, P) >= 2048) return P;
  return 256;
}

// Checks that need nothing but the descriptor.
attn_status check_desc(const attn_desc* d) {
  if (d == nullptr) return ATTN_ERR_NULL;
  if (d->num_seqs < 0 || d->num_tokens < 0 || d->num_decodes < 0 || d->max_query_len < 0 ||
      d->max_seq_len < 0 || d->num_heads <= 0 || d->num_kv_heads <= 0 || d->num_blocks < 0 ||
      d->max_blocks_per_seq < 0 || d->num_decodes > d->num_seqs ||
      d->max_query_len > d->max_seq_len)
    return ATTN_ERR_SHAPE;
  if (d->block_size <= 0 || d->block_size % 16 != 0) return ATTN_ERR_BLOCK_SIZE;
  if (d->num_heads % d->num_kv_heads != 0) return ATTN_ERR_GQA;
  if (d->head_size != 64 && d->head_size != 128) return ATTN_ERR_UNSUPPORTED;
  if (d->dtype != ATTN_BF16 && d->dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if (d->partition_tokens < 0 || d->partition_tokens > attn::kMaxPartitionTokens ||
      (d->partition_tokens > 0 && d->partition_tokens % 128 != 0))
    return ATTN_ERR_UNSUPPORTED;
  if (d->num_seqs > 65535) return ATTN_ERR_SHAPE;                    // grid z limit
  if (ceil_div(d->max_query_len, 256) > 65535) return ATTN_ERR_SHAPE;  // q tiles: grid z limit
  if ((int64_t)d->max_seq_len > (int64_t)d->max_blocks_per_seq * d->block_size)
    return ATTN_ERR_SHAPE;
  if ((int64_t)d->max_seq_len * d->block_size >= ((int64_t)1 << 40)) return ATTN_ERR_SHAPE;
  if ((int64_t)d->block_size * d->num_kv_heads * d->head_size >= ((int64_t)1 << 31))
    return ATTN_ERR_SHAPE;                                            // one block < 2^31 elements
  // decode partitions per request, and the split kernel's 1-D grid of (request, partition,
  // kv head, head group) workgroups
  if (ceil_div(d->max_seq_len, partition_tokens(d)) > 65535) return ATTN_ERR_SHAPE;
  if ((int64_t)d->num_decodes * ceil_div(d->max_seq_len, partition_tokens(d)) * d->num_kv_heads *
          ceil_div(d->num_heads / d->num_kv_heads, 16) >= ((int64_t)1 << 31))
    return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

bool uses_split_decode(const attn_desc* d) { return d->dtype == ATTN_BF16 && d->num_decodes > 0; }

// Partitions a decode request may span: all of max_seq_len, or with a window at most
// ceil(window / P) + 1 of them.
int64_t decode_max_parts(const attn_desc* d, int32_t window) {
  const int64_t P = partition_tokens(d);
  int64_t n = ceil_div(d->max_seq_len, P);
  if (window > 0) {
    const int64_t wn = ceil_div(window, P) + 1;
    if (wn < n) n = wn;
  }
  return n < 1 ? 1 : n;
}

// Decode work items (segments) a request may span, capped for a window like the partitions.
int64_t decode_max_segs(const attn_desc* d, int32_t window) {
  const int64_t S = attn::decode_segment_tokens(partition_tokens(d));
  int64_t n = ceil_div(d->max_seq_len, S);
  if (window > 0) {
    const int64_t wn = ceil_div(window, S) + 1;
    if (wn < n) n = wn;
  }
  return n < 1 ? 1 : n;
}

// Split-KV workspace: the partitions' results ([num_decodes][Hq][max_parts][d] bf16, then
// [num_decodes][Hq][max_parts] fp32 log-sum-exps), then, from a 256-byte boundary, the decode
// schedule region (below).
int64_t decode_results_bytes(const attn_desc* d, int64_t max_parts) {
  const int64_t rows = (int64_t)d->num_decodes * d->num_heads * max_parts;
  return ceil_div(rows * d->head_size * 2 + rows * 4, 256) * 256;
}
// Decode schedule region: the item count, then one int32 per (request, partition) slot.
int64_t decode_schedule_ints(const attn_desc* d, int64_t max_parts) {
  return 1 + (int64_t)d->num_decodes * max_parts;
}
size_t workspace_for(const attn_desc* d, int64_t max_parts) {
  if (!uses_split_decode(d)) return 0;
  return (size_t)(decode_results_bytes(d, max_parts) +
                  ceil_div(decode_schedule_ints(d, max_parts) * 4, 256) * 256);
}

size_t round256(int64_t bytes) { return (size_t)ceil_div(bytes, 256) * 256; }

// Key slices of the cascade prefix pass. Its rows are the (token, q head) pairs of each GQA
// group, 256 per workgroup; with few rows the prefix keys are split into slices (at least 512
// keys each, a multiple of the prefill kernel's key tile: 128 keys for head_size 128, 64 for
// 64) until about 512 workgroups run.
struct PrefixSplit {
  int32_t slices, slice_keys;
};
PrefixSplit prefix_split(const attn_desc* d, int32_t prefix) {
  const int64_t rows = (int64_t)d->num_tokens * (d->num_heads / d->num_kv_heads);
  const int64_t wgs = ceil_div(rows, 256) * d->num_kv_heads;
  int64_t s = ceil_div(512, wgs);
  const int64_t max_s = ceil_div(prefix, 512);
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  const int64_t tile = d->head_size == 128 ? 128 : 64;
  const int64_t keys = ceil_div(ceil_div(prefix, s), tile) * tile;
  return {(int32_t)ceil_div(prefix, keys), (int32_t)keys};
}

// Cascade workspace: the prefix pass's fp32 partial result for every query row
// ([num_tokens][Hq][d], then [num_tokens][Hq] log-sum-exps); with key slices, the slices'
// partial results in the same layout, slice after slice; then the decode partitions'
// workspace of the suffix pass.
size_t cascade_prefix_bytes(const attn_desc* d, int32_t prefix) {
  const int64_t rows = (int64_t)d->num_tokens * d->num_heads;
  const PrefixSplit sp = prefix_split(d, prefix);
  const int64_t copies = sp.slices > 1 ? 1 + sp.slices : 1;
  return copies * (round256(rows * d->head_size * 4) + round256(rows * 4));
}

attn::PrefillParams prefill_params(const attn_desc& d, const void* q, const void* kv_cache,
                                   const int32_t* block_table, const int32_t* qsl,
                                   const int32_t* seq_lens, float scale, int32_t causal,
                                   int32_t window, void* out, float* lse) {
  attn::PrefillParams pp{};
  pp.q = q;
  pp.kv = kv_cache;
  pp.block_table = block_table;
  pp.qsl = qsl;
  pp.seq_lens = seq_lens;
  pp.out = out;
  pp.lse = lse;
  pp.v_offset = (int64_t)d.num_blocks * d.block_size * d.num_kv_heads * d.head_size;
  pp.num_heads = d.num_heads;
  pp.num_kv_heads = d.num_kv_heads;
  pp.head_size = d.head_size;
  pp.block_size = d.block_size;
  pp.max_blocks = d.max_blocks_per_seq;
  pp.max_query_len = d.max_query_len;
  pp.causal = causal ? 1 : 0;
  pp.window = window > 0 ? window : 0;
  pp.scale = scale;
  const uint64_t groups = (uint64_t)(d.block_size / 16);
  pp.group_recip = (((uint64_t)1 << 32) + groups - 1) / groups;
  return pp;
}

attn::DecodeParams decode_params(const attn_desc& d, const attn::PrefillParams& pp,
                                 int64_t max_parts, float* ws) {
  attn::DecodeParams dp{};
  dp.q = pp.q;
  dp.kv = pp.kv;
  dp.block_table = pp.block_table;
  dp.qsl = pp.qsl;
  dp.seq_lens = pp.seq_lens;
  dp.out = pp.out;
  dp.lse = pp.lse;
  const int64_t rows = (int64_t)d.num_decodes * d.num_heads * max_parts;
  dp.ws_o = reinterpret_cast<__bf16*>(ws);
  dp.ws_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + rows * d.head_size * 2);
  dp.v_offset = pp.v_offset;
  dp.num_heads = d.num_heads;
  dp.num_kv_heads = d.num_kv_heads;
  dp.head_size = d.head_size;
  dp.block_size = d.block_size;
  dp.max_blocks = d.max_blocks_per_seq;
  dp.num_decodes = d.num_decodes;
  dp.part_tokens = partition_tokens(&d);
  dp.max_parts = (int32_t)max_parts;
  dp.seg_tokens = attn::decode_segment_tokens(dp.part_tokens);
  dp.max_segs = (int32_t)decode_max_segs(&d, pp.window);
  dp.schedule = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) +
                                           decode_results_bytes(&d, max_parts));
  dp.window = pp.window;
  dp.scale = pp.scale;
  dp.group_recip = pp.group_recip;
  return dp;
}

// Decode schedule region built ahead of a call, for the window's partition cap.
size_t decode_schedule_bytes_for(const attn_desc* d, int32_t window) {
  return round256(decode_schedule_ints(d, decode_max_parts(d, window)) * 4);
}

// Prefill work schedule: one int32 count plus one int32 per (prefill request, q tile) slot.
int64_t schedule_max_qtiles(const attn_desc* d) { return ceil_div(d->max_query_len, 256); }
size_t schedule_bytes_for(const attn_desc* d) {
  const int64_t slots = (int64_t)(d->num_seqs - d->num_decodes) * schedule_max_qtiles(d);
  return round256((1 + slots) * 4);
}

// Checks of a cascade call that need nothing but the descriptor and the prefix length.
attn_status check_cascade(const attn_desc* d, int32_t common_prefix_len) {
  const attn_status s = check_desc(d);
  if (s != ATTN_OK) return s;
  if (d->dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (common_prefix_len < 0 || common_prefix_len % d->block_size != 0 ||
      common_prefix_len > d->max_seq_len)
    return ATTN_ERR_SHAPE;
  if ((int64_t)d->num_tokens * d->num_heads >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status attn_workspace_bytes(const attn_desc* desc, size_t* bytes) {
  if (bytes == nullptr) return ATTN_ERR_NULL;
  const attn_status s = check_desc(desc);
  if (s != ATTN_OK) return s;
  *bytes = workspace_for(desc, decode_max_parts(desc, 0));
  return ATTN_OK;
}

attn_status attn_decode_partition_tokens(const attn_desc* desc, int32_t* tokens) {
  if (tokens == nullptr) return ATTN_ERR_NULL;
  const attn_status s = check_desc(desc);
  if (s != ATTN_OK) return s;
  *tokens = partition_tokens(desc);
  return ATTN_OK;
}

attn_status attn_varlen_fwd(const attn_desc* desc, const void* q, const void* kv_cache,
                            const int32_t* block_table, const int32_t* query_start_loc,
                            const int32_t* seq_lens, float scale, int32_t causal,
                            int32_t window, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream) {
  attn_status s = check_desc(desc);
  if (s != ATTN_OK) return s;
  const attn_desc& d = *desc;
  if (window > 0 && !causal) return ATTN_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !std::isfinite(scale)) return ATTN_ERR_UNSUPPORTED;
  if (d.num_seqs == 0 || d.num_tokens == 0) return ATTN_OK;
  if (q == nullptr || kv_cache == nullptr || block_table == nullptr ||
      query_start_loc == nullptr || seq_lens == nullptr || out == nullptr)
    return ATTN_ERR_NULL;

  const int64_t max_parts = decode_max_parts(&d, window);
  const size_t need = workspace_for(&d, max_parts);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  attn::PrefillParams pp = prefill_params(d, q, kv_cache, block_table, query_start_loc,
                                          seq_lens, scale, causal, window, out, lse);
  if (d.dtype == ATTN_F32) {
    // float32 runs every request, decode rows included, through the fp32 prefill kernel
    pp.seq_begin = 0;
    pp.num_seqs = d.num_seqs;
    return attn::launch_prefill_f32(pp, st) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
  }
  if (d.num_decodes > 0) {
    const attn::DecodeParams dp =
        decode_params(d, pp, max_parts, static_cast<float*>(workspace));
    if (attn::launch_decode_bf16(dp, st) != hipSuccess) return ATTN_ERR_HIP;
  }
  if (d.num_seqs > d.num_decodes) {
    pp.seq_begin = d.num_decodes;
    pp.num_seqs = d.num_seqs - d.num_decodes;
    if (attn::launch_prefill_bf16(pp, st) != hipSuccess) return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

attn_status attn_varlen_fwd_noalloc(const attn_desc* desc, const void* q, const void* kv_cache,
                                    const int32_t* block_table,
                                    const int32_t* query_start_loc, const int32_t* seq_lens,
                                    float scale, int32_t causal, int32_t window, void* out,
                                    float* lse, void* stream) {
  const attn_status s = check_desc(desc);
  if (s != ATTN_OK) return s;
  // the same checks attn_varlen_fwd makes, before the workspace size is looked at
  if (window > 0 && !causal) return ATTN_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !std::isfinite(scale)) return ATTN_ERR_UNSUPPORTED;
  if (desc->num_seqs == 0 || desc->num_tokens == 0) return ATTN_OK;
  if (q == nullptr || kv_cache == nullptr || block_table == nullptr ||
      query_start_loc == nullptr || seq_lens == nullptr || out == nullptr)
    return ATTN_ERR_NULL;
  const size_t need = workspace_for(desc, decode_max_parts(desc, window));
  if (need > (size_t)ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    const attn_status a = scratch_address(&ws);
    if (a != ATTN_OK) return a;
  }
  return attn_varlen_fwd(desc, q, kv_cache, block_table, query_start_loc, seq_lens, scale,
                         causal, window, out, lse, ws, need > 0 ? (size_t)ATTN_NOALLOC_SCRATCH_BYTES
                                                                : 0,
                         stream);
}

attn_status attn_cascade_workspace_bytes(const attn_desc* desc, int32_t common_prefix_len,
                                         size_t* bytes) {
  if (bytes == nullptr) return ATTN_ERR_NULL;
  const attn_status s = check_cascade(desc, common_prefix_len);
  if (s != ATTN_OK) return s;
  const size_t suffix = workspace_for(desc, decode_max_parts(desc, 0));
  *bytes = common_prefix_len == 0 ? suffix : cascade_prefix_bytes(desc, common_prefix_len) + suffix;
  return ATTN_OK;
}

attn_status attn_cascade_fwd(const attn_desc* desc, const void* q, const void* kv_cache,
                             const int32_t* block_table, const int32_t* query_start_loc,
                             const int32_t* seq_lens, int32_t common_prefix_len, float scale,
                             int32_t causal, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  attn_status s = check_cascade(desc, common_prefix_len);
  if (s != ATTN_OK) return s;
  if (common_prefix_len == 0)
    return attn_varlen_fwd(desc, q, kv_cache, block_table, query_start_loc, seq_lens, scale,
                           causal, 0, out, lse, workspace, workspace_bytes, stream);
  const attn_desc& d = *desc;
  if (!(scale > 0.f) || !std::isfinite(scale)) return ATTN_ERR_UNSUPPORTED;
  if (d.num_seqs == 0 || d.num_tokens == 0) return ATTN_OK;
  if (q == nullptr || kv_cache == nullptr || block_table == nullptr ||
      query_start_loc == nullptr || seq_lens == nullptr || out == nullptr)
    return ATTN_ERR_NULL;
  const int64_t max_parts = decode_max_parts(&d, 0);
  const size_t pre_bytes = cascade_prefix_bytes(&d, common_prefix_len);
  const size_t need = pre_bytes + workspace_for(&d, max_parts);
  if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t rows = (int64_t)d.num_tokens * d.num_heads;
  const size_t copy_bytes = round256(rows * d.head_size * 4) + round256(rows * 4);
  char* const wsb = static_cast<char*>(workspace);
  float* pre_o = reinterpret_cast<float*>(wsb);
  float* pre_lse = reinterpret_cast<float*>(wsb + round256(rows * d.head_size * 4));
  float* ws_suffix = reinterpret_cast<float*>(wsb + pre_bytes);
  const int32_t skip = common_prefix_len / d.block_size;
  const PrefixSplit sp = prefix_split(&d, common_prefix_len);

  // 1. prefix pass: every query token of the batch against the shared prefix, no mask;
  //    with key slices, each slice's partial result goes to its own copy, merged afterwards
  attn::PrefillParams pre = prefill_params(d, q, kv_cache, block_table, query_start_loc,
                                           seq_lens, scale, 0, 0, nullptr, pre_lse);
  pre.single_ql = d.num_tokens;
  pre.single_sl = common_prefix_len;
  pre.num_seqs = 1;
  pre.out_f32 = pre_o;
  if (sp.slices > 1) {
    pre.single_slice = sp.slice_keys;
    pre.slice_stride = rows;
    pre.out_f32 = reinterpret_cast<float*>(wsb + copy_bytes);
    pre.lse = reinterpret_cast<float*>(wsb + copy_bytes + (size_t)sp.slices *
                                       round256(rows * d.head_size * 4));
  }
  if (attn::launch_prefill_bf16(pre, st) != hipSuccess) return ATTN_ERR_HIP;
  if (sp.slices > 1) {
    attn::PrefixMergeParams mp{};
    mp.o_in = pre.out_f32;
    mp.lse_in = pre.lse;
    mp.o_out = pre_o;
    mp.lse_out = pre_lse;
    mp.rows = rows;
    mp.slices = sp.slices;
    if (attn::launch_prefix_slices_merge(mp, d.head_size, st) != hipSuccess) return ATTN_ERR_HIP;
  }

  // 2. suffix pass over the keys after the prefix, merged with the prefix result
  attn::PrefillParams pp = prefill_params(d, q, kv_cache, block_table, query_start_loc,
                                          seq_lens, scale, causal, 0, out, lse);
  pp.kv_skip_blocks = skip;
  if (d.num_decodes > 0) {
    attn::DecodeParams dp = decode_params(d, pp, max_parts, ws_suffix);
    dp.kv_skip_blocks = skip;
    dp.pre_o = pre_o;
    dp.pre_lse = pre_lse;
    if (attn::launch_decode_bf16(dp, st) != hipSuccess) return ATTN_ERR_HIP;
  }
  if (d.num_seqs > d.num_decodes) {
    pp.seq_begin = d.num_decodes;
    pp.num_seqs = d.num_seqs - d.num_decodes;
    pp.init_o = pre_o;
    pp.init_lse = pre_lse;
    if (attn::launch_prefill_bf16(pp, st) != hipSuccess) return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

attn_status attn_check_cascade_host(const attn_desc* desc, const int32_t* block_table,
                                    const int32_t* query_start_loc, const int32_t* seq_lens,
                                    int32_t common_prefix_len) {
  attn_status s = check_cascade(desc, common_prefix_len);
  if (s != ATTN_OK) return s;
  s = attn_check_metadata_host(desc, block_table, query_start_loc, seq_lens);
  if (s != ATTN_OK) return s;
  const attn_desc& d = *desc;
  const int64_t nb = common_prefix_len / d.block_size;
  for (int32_t r = 0; r < d.num_seqs; ++r) {
    const int64_t ql = (int64_t)query_start_loc[r + 1] - query_start_loc[r];
    if ((int64_t)seq_lens[r] - ql < common_prefix_len) return ATTN_ERR_METADATA;
    for (int64_t b = 0; b < nb; ++b)
      if (block_table[(int64_t)r * d.max_blocks_per_seq + b] != block_table[b])
        return ATTN_ERR_METADATA;
  }
  return ATTN_OK;
}

attn_status attn_schedule_bytes(const attn_desc* desc, size_t* bytes) {
  if (bytes == nullptr) return ATTN_ERR_NULL;
  const attn_status s = check_desc(desc);
  if (s != ATTN_OK) return s;
  if ((int64_t)(desc->num_seqs - desc->num_decodes) * schedule_max_qtiles(desc) *
          desc->num_heads >= ((int64_t)1 << 31))
    return ATTN_ERR_SHAPE;
  *bytes = schedule_bytes_for(desc);
  return ATTN_OK;
}

attn_status attn_build_schedule(const attn_desc* desc, const int32_t* query_start_loc,
                                const int32_t* seq_lens, int32_t causal, int32_t window,
                                int32_t* schedule, size_t schedule_bytes, void* stream) {
  size_t need = 0;
  const attn_status s = attn_schedule_bytes(desc, &need);
  if (s != ATTN_OK) return s;
  if (window > 0 && !causal) return ATTN_ERR_UNSUPPORTED;
  if (schedule == nullptr || schedule_bytes < need) return ATTN_ERR_WORKSPACE;
  if (desc->num_seqs > desc->num_decodes && (query_start_loc == nullptr || seq_lens == nullptr))
    return ATTN_ERR_NULL;
  attn::ScheduleParams sp{};
  sp.qsl = query_start_loc;
  sp.seq_lens = seq_lens;
  sp.schedule = schedule;
  sp.seq_begin = desc->num_decodes;
  sp.num_seqs = desc->num_seqs - desc->num_decodes;
  sp.max_qtiles = (int32_t)schedule_max_qtiles(desc);
  sp.causal = causal ? 1 : 0;
  sp.window = window > 0 ? window : 0;
  return attn::launch_prefill_schedule(sp, static_cast<hipStream_t>(stream)) == hipSuccess
             ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_varlen_fwd_scheduled(const attn_desc* desc, const void* q, const void* kv_cache,
                                      const int32_t* block_table,
                                      const int32_t* query_start_loc, const int32_t* seq_lens,
                                      float scale, int32_t causal, int32_t window, void* out,
                                      float* lse, void* workspace, size_t workspace_bytes,
                                      const int32_t* schedule, size_t schedule_bytes,
                                      void* stream) {
  attn_status s = check_desc(desc);
  if (s != ATTN_OK) return s;
  const attn_desc& d = *desc;
  if (d.dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  size_t need_sched = 0;
  s = attn_schedule_bytes(desc, &need_sched);
  if (s != ATTN_OK) return s;
  if (window > 0 && !causal) return ATTN_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !std::isfinite(scale)) return ATTN_ERR_UNSUPPORTED;
  if (d.num_seqs == 0 || d.num_tokens == 0) return ATTN_OK;
  if (q == nullptr || kv_cache == nullptr || block_table == nullptr ||
      query_start_loc == nullptr || seq_lens == nullptr || out == nullptr)
    return ATTN_ERR_NULL;
  if (schedule == nullptr || schedule_bytes < need_sched) return ATTN_ERR_WORKSPACE;
  const int64_t max_parts = decode_max_parts(&d, window);
  const size_t need = workspace_for(&d, max_parts);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  attn::PrefillParams pp = prefill_params(d, q, kv_cache, block_table, query_start_loc,
                                          seq_lens, scale, causal, window, out, lse);
  if (d.num_decodes > 0) {
    const attn::DecodeParams dp =
        decode_params(d, pp, max_parts, static_cast<float*>(workspace));
    if (attn::launch_decode_bf16(dp, st) != hipSuccess) return ATTN_ERR_HIP;
  }
  if (d.num_seqs > d.num_decodes) {
    pp.seq_begin = d.num_decodes;
    pp.num_seqs = d.num_seqs - d.num_decodes;
    pp.schedule = schedule;
    pp.max_qtiles = (int32_t)schedule_max_qtiles(&d);
    if (attn::launch_prefill_bf16(pp, st) != hipSuccess) return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

attn_status attn_decode_schedule_bytes(const attn_desc* desc, int32_t window, size_t* bytes) {
  if (bytes == nullptr) return ATTN_ERR_NULL;
  const attn_status s = check_desc(desc);
  if (s != ATTN_OK) return s;
  *bytes = uses_split_decode(desc) ? decode_schedule_bytes_for(desc, window) : 0;
  return ATTN_OK;
}

attn_status attn_build_decode_schedule(const attn_desc* desc, const int32_t* seq_lens,
                                       int32_t window, int32_t* schedule,
                                       size_t schedule_bytes, void* stream) {
  size_t need = 0;
  const attn_status s = attn_decode_schedule_bytes(desc, window, &need);
  if (s != ATTN_OK) return s;
  if (need == 0) return ATTN_OK;                 // no split-KV decode rows: nothing to build
  if (schedule == nullptr || schedule_bytes < need) return ATTN_ERR_WORKSPACE;
  if (seq_lens == nullptr) return ATTN_ERR_NULL;
  attn::DecodeScheduleParams sp{};
  sp.seq_lens = seq_lens;
  sp.schedule = schedule;
  sp.num_decodes = desc->num_decodes;
  sp.part_tokens = attn::decode_segment_tokens(partition_tokens(desc));
  sp.max_parts = (int32_t)decode_max_segs(desc, window);
  sp.window = window > 0 ? window : 0;
  sp.kv_skip_keys = 0;
  return attn::launch_decode_schedule(sp, static_cast<hipStream_t>(stream)) == hipSuccess
             ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_varlen_fwd_prescheduled(
    const attn_desc* desc, const void* q, const void* kv_cache, const int32_t* block_table,
    const int32_t* query_start_loc, const int32_t* seq_lens, float scale, int32_t causal,
    int32_t window, void* out, float* lse, void* workspace, size_t workspace_bytes,
    const int32_t* prefill_schedule, size_t prefill_schedule_bytes,
    const int32_t* decode_schedule, size_t decode_schedule_bytes, void* stream) {
  attn_status s = check_desc(desc);
  if (s != ATTN_OK) return s;
  const attn_desc& d = *desc;
  if (window > 0 && !causal) return ATTN_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !std::isfinite(scale)) return ATTN_ERR_UNSUPPORTED;
  if (prefill_schedule != nullptr) {
    if (d.dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    size_t need_sched = 0;
    s = attn_schedule_bytes(desc, &need_sched);
    if (s != ATTN_OK) return s;
    if (prefill_schedule_bytes < need_sched) return ATTN_ERR_WORKSPACE;
  }
  if (decode_schedule != nullptr && uses_split_decode(&d) &&
      decode_schedule_bytes < decode_schedule_bytes_for(&d, window))
    return ATTN_ERR_WORKSPACE;
  if (d.num_seqs == 0 || d.num_tokens == 0) return ATTN_OK;
  if (q == nullptr || kv_cache == nullptr || block_table == nullptr ||
      query_start_loc == nullptr || seq_lens == nullptr || out == nullptr)
    return ATTN_ERR_NULL;
  const int64_t max_parts = decode_max_parts(&d, window);
  const size_t need = workspace_for(&d, max_parts);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  attn::PrefillParams pp = prefill_params(d, q, kv_cache, block_table, query_start_loc,
                                          seq_lens, scale, causal, window, out, lse);
  if (d.dtype == ATTN_F32) {
    pp.seq_begin = 0;
    pp.num_seqs = d.num_seqs;
    return attn::launch_prefill_f32(pp, st) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
  }
  if (d.num_decodes > 0) {
    attn::DecodeParams dp = decode_params(d, pp, max_parts, static_cast<float*>(workspace));
    dp.items = decode_schedule;                   // null: the launch builds it in the workspace
    if (attn::launch_decode_bf16(dp, st) != hipSuccess) return ATTN_ERR_HIP;
  }
  if (d.num_seqs > d.num_decodes) {
    pp.seq_begin = d.num_decodes;
    pp.num_seqs = d.num_seqs - d.num_decodes;
    if (prefill_schedule != nullptr) {
      pp.schedule = prefill_schedule;
      pp.max_qtiles = (int32_t)schedule_max_qtiles(&d);
    }
    if (attn::launch_prefill_bf16(pp, st) != hipSuccess) return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

attn_status attn_varlen_fwd_mixed(const attn_desc* desc, const void* q, const void* kv_cache,
                                  const int32_t* block_table, const int32_t* query_start_loc,
                                  const int32_t* seq_lens, float scale, int32_t causal,
                                  int32_t window, void* out, float* lse,
                                  const int32_t* prefill_schedule, size_t prefill_schedule_bytes,
                                  void* stream) {
  attn_status s = check_desc(desc);
  if (s != ATTN_OK) return s;
  const attn_desc& d = *desc;
  if (d.dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (window > 0 && !causal) return ATTN_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !std::isfinite(scale)) return ATTN_ERR_UNSUPPORTED;
  size_t need_sched = 0;
  s = attn_schedule_bytes(desc, &need_sched);
  if (s != ATTN_OK) return s;
  const bool has_prefill = d.num_seqs > d.num_decodes;
  if (has_prefill && (prefill_schedule == nullptr || prefill_schedule_bytes < need_sched))
    return ATTN_ERR_WORKSPACE;
  if (d.num_seqs == 0 || d.num_tokens == 0) return ATTN_OK;
  if (q == nullptr || kv_cache == nullptr || block_table == nullptr ||
      query_start_loc == nullptr || seq_lens == nullptr || out == nullptr)
    return ATTN_ERR_NULL;
  attn::PrefillParams pp = prefill_params(d, q, kv_cache, block_table, query_start_loc,
                                          seq_lens, scale, causal, window, out, lse);
  const attn::DecodeParams dp = decode_params(d, pp, 1, nullptr);   // no partials: no workspace
  pp.seq_begin = d.num_decodes;
  pp.num_seqs = has_prefill ? d.num_seqs - d.num_decodes : 0;
  pp.schedule = prefill_schedule;
  pp.max_qtiles = (int32_t)schedule_max_qtiles(&d);
  return attn::launch_mixed_bf16(pp, dp, static_cast<hipStream_t>(stream)) == hipSuccess
             ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_check_metadata_host(const attn_desc* desc, const int32_t* block_table,
                                     const int32_t* query_start_loc, const int32_t* seq_lens) {
  const attn_status s = check_desc(desc);
  if (s != ATTN_OK) return s;
  const attn_desc& d = *desc;
  if (d.num_seqs == 0) return d.num_tokens == 0 ? ATTN_OK : ATTN_ERR_METADATA;
  if (block_table == nullptr || query_start_loc == nullptr || seq_lens == nullptr)
    return ATTN_ERR_NULL;
  if (query_start_loc[0] != 0 || query_start_loc[d.num_seqs] != d.num_tokens)
    return ATTN_ERR_METADATA;
  for (int32_t r = 0; r < d.num_seqs; ++r) {
    const int64_t ql = (int64_t)query_start_loc[r + 1] - query_start_loc[r];
    const int64_t sl = seq_lens[r];
    if (ql < 0 || sl < ql || sl > d.max_seq_len || ql > d.max_query_len) return ATTN_ERR_METADATA;
    if (r < d.num_decodes && ql != 1) return ATTN_ERR_METADATA;
    const int64_t nb = ceil_div(sl, d.block_size);
    if (nb > d.max_blocks_per_seq) return ATTN_ERR_METADATA;
    for (int64_t b = 0; b < nb; ++b) {
      const int32_t blk = block_table[(int64_t)r * d.max_blocks_per_seq + b];
      if (blk < 0 || blk >= d.num_blocks) return ATTN_ERR_METADATA;
    }
  }
  return ATTN_OK;
}

attn_status attn_kv_cache_write(const attn_desc* desc, const void* key, int64_t key_row_stride,
                                const void* value, int64_t value_row_stride,
                                const int64_t* slot_mapping, void* kv_cache, void* stream) {
  if (desc == nullptr) return ATTN_ERR_NULL;
  const attn_desc& d = *desc;
  if (d.num_tokens < 0 || d.num_kv_heads <= 0 || d.num_blocks < 0) return ATTN_ERR_SHAPE;
  if (d.block_size <= 0 || d.block_size % 16 != 0) return ATTN_ERR_BLOCK_SIZE;
  if (d.head_size != 64 && d.head_size != 128) return ATTN_ERR_UNSUPPORTED;
  if (d.dtype != ATTN_BF16 && d.dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  const int64_t elem = d.dtype == ATTN_BF16 ? 2 : 4;
  const int64_t row = (int64_t)d.num_kv_heads * d.head_size;        // elements per token row
  if (key_row_stride < row || value_row_stride < row) return ATTN_ERR_SHAPE;
  // 16-byte chunks: rows must start on 16-byte boundaries
  if ((key_row_stride * elem) % 16 != 0 || (value_row_stride * elem) % 16 != 0)
    return ATTN_ERR_SHAPE;
  if ((int64_t)d.num_tokens * 2 * (row * elem / 16) / 256 >= ((int64_t)1 << 31))
    return ATTN_ERR_SHAPE;                                          // grid x limit
  if (d.num_tokens == 0) return ATTN_OK;
  if (key == nullptr || value == nullptr || slot_mapping == nullptr || kv_cache == nullptr)
    return ATTN_ERR_NULL;
  if ((uintptr_t)key % 16 != 0 || (uintptr_t)value % 16 != 0 || (uintptr_t)kv_cache % 16 != 0)
    return ATTN_ERR_SHAPE;
  attn::KvWriteParams p{};
  p.key = key;
  p.value = value;
  p.slot_mapping = slot_mapping;
  p.kv_cache = kv_cache;
  p.num_tokens = d.num_tokens;
  p.key_stride_bytes = key_row_stride * elem;
  p.value_stride_bytes = value_row_stride * elem;
  p.slot_bytes = row * elem;
  p.row_chunks = p.slot_bytes / 16;
  p.num_slots = (int64_t)d.num_blocks * d.block_size;
  p.v_offset_bytes = p.num_slots * p.slot_bytes;
  return attn::launch_kv_write(p, static_cast<hipStream_t>(stream)) == hipSuccess ? ATTN_OK
                                                                                : ATTN_ERR_HIP;
}

attn_status attn_kv_cache_write_fp8(const attn_desc* desc, const void* key,
                                    int64_t key_row_stride, const void* value,
                                    int64_t value_row_stride, const int64_t* slot_mapping,
                                    float k_scale, float v_scale, void* kv_cache, void* stream) {
  if (desc == nullptr) return ATTN_ERR_NULL;
  const attn_desc& d = *desc;
  if (d.num_tokens < 0 || d.num_kv_heads <= 0 || d.num_blocks < 0) return ATTN_ERR_SHAPE;
  if (d.block_size <= 0 || d.block_size % 16 != 0) return ATTN_ERR_BLOCK_SIZE;
  if (d.head_size != 64 && d.head_size != 128) return ATTN_ERR_UNSUPPORTED;
  if (d.dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;          // bf16 rows in, codes out
  if (!(k_scale > 0.f) || !std::isfinite(k_scale) || !(v_scale > 0.f) || !std::isfinite(v_scale))
    return ATTN_ERR_UNSUPPORTED;
  const int64_t row = (int64_t)d.num_kv_heads * d.head_size;        // elements per token row
  if (key_row_stride < row || value_row_stride < row) return ATTN_ERR_SHAPE;
  if ((key_row_stride * 2) % 16 != 0 || (value_row_stride * 2) % 16 != 0) return ATTN_ERR_SHAPE;
  if ((int64_t)d.num_tokens * 2 * (row / 16) / 256 >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
  if (d.num_tokens == 0) return ATTN_OK;
  if (key == nullptr || value == nullptr || slot_mapping == nullptr || kv_cache == nullptr)
    return ATTN_ERR_NULL;
  if ((uintptr_t)key % 16 != 0 || (uintptr_t)value % 16 != 0 || (uintptr_t)kv_cache % 16 != 0)
    return ATTN_ERR_SHAPE;
  attn::KvWriteParams p{};
  p.key = key;
  p.value = value;
  p.slot_mapping = slot_mapping;
  p.kv_cache = kv_cache;
  p.num_tokens = d.num_tokens;
  p.key_stride_bytes = key_row_stride * 2;
  p.value_stride_bytes = value_row_stride * 2;
  p.slot_bytes = row;                                               // one code per element
  p.row_chunks = row / 16;
  p.num_slots = (int64_t)d.num_blocks * d.block_size;
  p.v_offset_bytes = p.num_slots * p.slot_bytes;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  return attn::launch_kv_write_fp8(p, static_cast<hipStream_t>(stream)) == hipSuccess
             ? ATTN_OK : ATTN_ERR_HIP;
}

// The E4M3 decode's partition when the descriptor leaves it to the library: the bf16 default
// capped at 1024 keys. Partitions of more than 1024 keys run one unit per 4-wave workgroup,
// and an E4M3 unit converts its codes and does the same MFMA and softmax work per key with
// half the bytes in flight per wave, so its latency shows; units of at most 1024 keys run one
// per wave (more independent streams per SIMD). Measured on gfx950: paged GQA decode (256
// requests of 512..8192 keys, 32 q / 8 kv heads) 59.6 % of 8 TB/s at the bf16 default (16384)
// against 71.2 % at 1024 keys; 120 requests of 4K..32K keys, 64 q / 8 kv heads, 62.6 % at 8192
// against 68.9 %. Kept at the bf16 default where 1024-key partitions would exceed the
// descriptor limits.
attn_desc fp8_decode_desc(const attn_desc& d) {
  attn_desc e = d;
  if (e.partition_tokens == 0) {
    e.partition_tokens = std::min(partition_tokens(&d), 1024);
    if (check_desc(&e) != ATTN_OK) e.partition_tokens = 0;
  }
  return e;
}

attn_status attn_fp8_decode_workspace_bytes(const attn_desc* desc, size_t* bytes) {
  if (bytes == nullptr) return ATTN_ERR_NULL;
  const attn_status s = check_desc(desc);
  if (s != ATTN_OK) return s;
  const attn_desc e = fp8_decode_desc(*desc);
  *bytes = workspace_for(&e, decode_max_parts(&e, 0));
  return ATTN_OK;
}

attn_status attn_fp8_decode_fwd(const attn_desc* desc, const void* q, const void* kv_cache,
                                const int32_t* block_table, const int32_t* query_start_loc,
                                const int32_t* seq_lens, float scale, float k_scale,
                                float v_scale, int32_t window, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream) {
  attn_status s = check_desc(desc);
  if (s != ATTN_OK) return s;
  const attn_desc d = fp8_decode_desc(*desc);
  if (d.dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;            // q and out are bf16
  if (d.num_decodes != d.num_seqs) return ATTN_ERR_UNSUPPORTED;     // decode rows only
  if (!(scale > 0.f) || !std::isfinite(scale) || !(k_scale > 0.f) || !std::isfinite(k_scale) ||
      !(v_scale > 0.f) || !std::isfinite(v_scale))
    return ATTN_ERR_UNSUPPORTED;
  if (d.num_seqs == 0 || d.num_tokens == 0) return ATTN_OK;
  if (q == nullptr || kv_cache == nullptr || block_table == nullptr ||
      query_start_loc == nullptr || seq_lens == nullptr || out == nullptr)
    return ATTN_ERR_NULL;
  const int64_t max_parts = decode_max_parts(&d, window);
  const size_t need = workspace_for(&d, max_parts);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  // k_scale multiplies every score: fold it into the softmax scale
  const attn::PrefillParams pp = prefill_params(d, q, kv_cache, block_table, query_start_loc,
                                                seq_lens, scale * k_scale, 1, window, out, lse);
  attn::DecodeParams dp = decode_params(d, pp, max_parts, static_cast<float*>(workspace));
  dp.v_scale = v_scale;
  return attn::launch_decode_fp8(dp, static_cast<hipStream_t>(stream)) == hipSuccess
             ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_check_slot_mapping_host(const attn_desc* desc, const int64_t* slot_mapping) {
  if (desc == nullptr) return ATTN_ERR_NULL;
  const attn_desc& d = *desc;
  if (d.num_tokens < 0 || d.num_blocks < 0) return ATTN_ERR_SHAPE;
  if (d.block_size <= 0 || d.block_size % 16 != 0) return ATTN_ERR_BLOCK_SIZE;
  if (d.num_tokens == 0) return ATTN_OK;
  if (slot_mapping == nullptr) return ATTN_ERR_NULL;
  const int64_t num_slots = (int64_t)d.num_blocks * d.block_size;
  std::vector<int64_t> seen;
  seen.reserve((size_t)d.num_tokens);
  for (int32_t t = 0; t < d.num_tokens; ++t) {
    const int64_t s = slot_mapping[t];
    if (s >= num_slots) return ATTN_ERR_METADATA;
    if (s >= 0) seen.push_back(s);
  }
  std::sort(seen.begin(), seen.end());
  for (size_t i = 1; i < seen.size(); ++i)
    if (seen[i] == seen[i - 1]) return ATTN_ERR_METADATA;
  return ATTN_OK;
}

const char* attn_status_str(int32_t status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_NULL: return "ATTN_ERR_NULL";
    case ATTN_ERR_SHAPE: return "ATTN_ERR_SHAPE";
    case ATTN_ERR_BLOCK_SIZE: return "ATTN_ERR_BLOCK_SIZE";
    case ATTN_ERR_GQA: return "ATTN_ERR_GQA";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    case ATTN_ERR_METADATA: return "ATTN_ERR_METADATA";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
    default: return "ATTN_ERR_UNKNOWN";
  }
}

}  // extern "C"
