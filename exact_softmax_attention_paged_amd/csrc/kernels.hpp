// Launch interface between the C-ABI layer and the gfx950 kernels (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Largest split-KV partition the decode kernel accepts (its block-id table holds
// kMaxPartitionTokens / 16 entries).
constexpr int32_t kMaxPartitionTokens = 16384;

// Keys of one decode work item (a segment of a request's keys). Partitions of up to
// kWaveSegmentTokens keys are streamed by one wave each, as many whole partitions per item as
// fit in kWaveSegmentTokens keys (the wave writes one partial result per partition); a longer
// partition is one item, streamed by one workgroup.
constexpr int32_t kWaveSegmentTokens = 1024;
__host__ __device__ inline int32_t decode_segment_tokens(int32_t part_tokens) {
  return part_tokens <= kWaveSegmentTokens ? kWaveSegmentTokens / part_tokens * part_tokens
                                           : part_tokens;
}

// One prefill launch covers requests [seq_begin, seq_begin + num_seqs) and every q head.
struct PrefillParams {
  const void* q;                // [num_tokens][num_heads][head_size]
  const void* kv;               // (2, num_blocks, block_size, num_kv_heads, head_size)
  const int32_t* block_table;   // [num_seqs_total][max_blocks]
  const int32_t* qsl;           // [num_seqs_total + 1]
  const int32_t* seq_lens;      // [num_seqs_total]
  void* out;
  float* lse;                   // may be null
  int64_t v_offset;             // elements between the K half and the V half
  int32_t num_heads, num_kv_heads, head_size, block_size, max_blocks;
  int32_t seq_begin, num_seqs, max_query_len;
  int32_t causal, window;
  float scale;
  uint64_t group_recip;         // ceil(2^32 / (block_size / 16)): block index of key k is
                                // ((k / 16) * group_recip) >> 32 for k * block_size < 2^40
  // Cascade passes (all zero / null for a plain call):
  int32_t kv_skip_blocks;       // keys start after this many blocks of every request (the
                                // shared prefix); seq_len shrinks by kv_skip_blocks*block_size
  int32_t single_ql, single_sl; // single_ql > 0: one sequence whose queries are rows
                                // [0, single_ql) of q and whose keys are the first single_sl
                                // keys of block-table row 0 (the prefix pass, no mask). Its
                                // rows are (token, q head) pairs of one kv head's GQA group
                                // (grid y = kv head), and grid z splits the keys into slices
                                // of single_slice keys (a multiple of the kernel's key tile:
                                // 128 for head_size 128, 64 for 64), slice z writing its
                                // partial result at out_f32 / lse + z * slice_stride rows
  int32_t single_slice;
  int64_t slice_stride;         // (token, head) rows between slices of out_f32 and lse
  float* out_f32;               // non-null: write O (normalised) in fp32 here, not to out
  const int32_t* schedule;      // non-null: grid x = item slot * num_heads + q head, items
                                // from a prefill schedule (see ScheduleParams)
  int32_t max_qtiles;           // q tiles per request in the schedule's item numbering
  const float* init_o;          // non-null: start each row from a partial result over
  const float* init_lse;        // earlier keys, fp32 [token][head][d] and [token][head]
};

// One split-KV decode launch covers requests [0, num_decodes): each has query_len == 1.
struct DecodeParams {
  const void* q;
  const void* kv;
  const int32_t* block_table;
  const int32_t* qsl;
  const int32_t* seq_lens;
  void* out;
  float* lse;
  __bf16* ws_o;                 // [num_decodes][num_heads][max_parts][head_size] partition
                                // results, normalised, rounded to bf16
  float* ws_lse;                // [num_decodes][num_heads][max_parts] their log-sum-exps
  int64_t v_offset;
  int32_t num_heads, num_kv_heads, head_size, block_size, max_blocks;
  int32_t num_decodes, part_tokens, max_parts;  // max_parts: partitions a request may span
  int32_t seg_tokens, max_segs; // work items: segments of decode_segment_tokens(part_tokens)
                                // keys; max_segs: segments a request may span
  int32_t window;
  float scale;
  uint64_t group_recip;         // ceil(2^32 / (block_size / 16)), as in PrefillParams
  float v_scale;                // E4M3 cache only: V dequantisation scale (k_scale is folded
                                // into scale by the host)
  int32_t* schedule;            // where the launch builds this call's work items (see
                                // DecodeScheduleParams), unless items is set
  const int32_t* items;         // the (request, segment) items the split kernel reads, longest
                                // first: schedule, or a schedule the caller built ahead (then
                                // nothing is built); unit = item slot * (num_kv_heads * head
                                // groups) + kv head group
  // Cascade suffix pass (zero / null for a plain call):
  int32_t kv_skip_blocks;       // as in PrefillParams
  const float* pre_o;           // non-null: a partial result over the prefix, fp32
  const float* pre_lse;         // [token][head][d] and [token][head], merged as one more
                                // partition (every row then goes through the merge kernel)
};

// Partitions of a decode request that hold visible keys: [first, first + count).
__host__ __device__ inline void decode_partitions(int32_t seq_len, int32_t window,
                                                  int32_t part_tokens, int32_t* first,
                                                  int32_t* count) {
  int32_t lo = window > 0 ? (seq_len - window > 0 ? seq_len - window : 0) : 0;
  int32_t f = lo / part_tokens;
  int32_t end = (seq_len + part_tokens - 1) / part_tokens;
  *first = f;
  *count = end > f ? end - f : 0;
}

// Merge of the key slices of the cascade prefix pass: rows = num_tokens * num_heads;
// slice z of row i is o_in[(z * rows + i) * d ..] and lse_in[z * rows + i].
struct PrefixMergeParams {
  const float* o_in;
  const float* lse_in;
  float* o_out;                 // [rows][d]
  float* lse_out;               // [rows]
  int64_t rows;
  int32_t slices;
};

// KV-cache write: token t's K row (key + t * key_stride_bytes) and V row go to slot
// slot_mapping[t] of the K and V halves of the cache.
struct KvWriteParams {
  const void* key;
  const void* value;
  const int64_t* slot_mapping;
  void* kv_cache;
  int64_t num_tokens;
  int64_t key_stride_bytes, value_stride_bytes;
  int64_t row_chunks;           // 16-byte chunks of one token's row (num_kv_heads * head_size)
  int64_t slot_bytes;           // bytes of one slot = one token's row
  int64_t num_slots;            // num_blocks * block_size
  int64_t v_offset_bytes;       // bytes from the K half to the V half
  float k_scale, v_scale;       // E4M3 cache only: code = E4M3(x / scale)
};

// Prefill work schedule: items (request, 256-row q tile) of requests
// [seq_begin, seq_begin + num_seqs), sorted by their number of 64-key tiles, longest first.
struct ScheduleParams {
  const int32_t* qsl;
  const int32_t* seq_lens;
  int32_t* schedule;            // [0] = item count, then the items
  int32_t seq_begin, num_seqs, max_qtiles;
  int32_t causal, window;
};

// Decode work schedule: items (decode request r, key range pi of part_tokens keys) coded
// r * max_parts + pi, for every range holding visible keys, sorted by their number of keys (in
// 16-key units), longest first, so the in-order workgroup dispatch leaves the short ranges to
// the end of the grid. schedule[0] = item count, schedule[1 + i] = item i. The decode kernel's
// items are its segments (part_tokens = its segment length, max_parts = its max_segs).
struct DecodeScheduleParams {
  const int32_t* seq_lens;
  int32_t* schedule;
  int32_t num_decodes, part_tokens, max_parts, window;
  int32_t kv_skip_keys;         // keys before the pass's range (cascade suffix pass)
};

hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream);
hipError_t launch_decode_schedule(const DecodeScheduleParams& p, hipStream_t stream);
hipError_t launch_prefill_schedule(const ScheduleParams& p, hipStream_t stream);
hipError_t launch_kv_write(const KvWriteParams& p, hipStream_t stream);
// E4M3 cache from bf16 rows: row_chunks counts 16-code chunks (slot_bytes = codes per row)
hipError_t launch_kv_write_fp8(const KvWriteParams& p, hipStream_t stream);
hipError_t launch_prefix_slices_merge(const PrefixMergeParams& p, int head_size,
                                      hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillParams& p, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_fp8(const DecodeParams& p, hipStream_t stream);   // E4M3 cache
// One launch for a mixed batch: decode requests [0, dp.num_decodes) one wave per (request, kv
// head group) over all their keys, and the prefill rows of p (p.schedule required).
hipError_t launch_mixed_bf16(const PrefillParams& p, const DecodeParams& dp, hipStream_t stream);

}  // namespace attn
