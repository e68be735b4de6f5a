/*
 * attn.h — C ABI of the MI355X (gfx950) exact paged attention library, libattn.so.
 *
 * The library computes exact scaled-dot-product attention over a paged KV cache for a
 * variable-length batch in one call, FlashAttention-style: scores are formed tile by tile,
 * the softmax is kept online (running max and running sum), partial results over KV
 * partitions are merged through their log-sum-exp, and the N x N score matrix never reaches
 * device memory.
 *
 * Sources (web pages this library follows; cited by title and section):
 *   [FA]   "[vLLM] FlashAttention: IO-aware 타일링으로 어텐션 연산을 가속하는 원리"
 *            - FlashAttentionBackend section: cache shape (2, num_blocks, block_size,
 *              num_kv_heads, head_size) and the block_size % 16 rule;
 *            - FlashAttentionImpl section: scale, num_kv_heads, num_queries_per_kv (GQA);
 *            - FlashAttentionMetadata section: query_start_loc, seq_lens, block_table,
 *              max_query_len, max_seq_len, one kernel call per varlen batch;
 *            - Intro and paper-summary sections: tiling plus online softmax, exactness.
 *   [RBLN] "Attention 모드" (RBLN vLLM docs): Overview (naive attention; partitions merged
 *              by online softmax), Full Attention (causal), Sliding-Window Attention.
 *   [OTH]  "[vLLM] 기타 Attention Backends ...", Triton Attention section:
 *              seq_len = context_len + query_len.
 *   [LIN]  "[vLLM] Lightning & Linear Attention ...", Prefill/Decode split section:
 *              requests with query_len == 1 are decode requests.
 *
 * Conventions for every entry point:
 *   - All tensors are caller-owned. Device pointers must stay valid until the work queued
 *     on `stream` has finished. The library never allocates, frees or synchronises device
 *     memory and keeps no global state (except the fixed device array of
 *     attn_varlen_fwd_noalloc); calls are thread-safe.
 *   - Errors are reported as attn_status codes. Argument errors are detected on the host
 *     before anything is queued, so a failed call leaves every buffer untouched.
 *   - Device-side metadata (block_table, query_start_loc, seq_lens) is trusted by
 *     attn_varlen_fwd: checking it would need a device-to-host synchronisation.
 *     attn_check_metadata_host validates host copies of it.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,       /* a size is negative or sizes are inconsistent */
  ATTN_ERR_BLOCK_SIZE = 3,  /* block_size is not a positive multiple of 16 ([FA] Backend) */
  ATTN_ERR_GQA = 4,         /* num_heads is not a multiple of num_kv_heads ([FA] Impl) */
  ATTN_ERR_UNSUPPORTED = 5, /* head_size, dtype, partition size or mask kind not built */
  ATTN_ERR_WORKSPACE = 6,   /* workspace missing or smaller than attn_workspace_bytes */
  ATTN_ERR_METADATA = 7,    /* attn_check_metadata_host found malformed metadata */
  ATTN_ERR_HIP = 8          /* a kernel launch failed */
} attn_status;

typedef enum attn_dtype {
  ATTN_BF16 = 0, /* q, kv_cache and out are bfloat16; accumulation is fp32 */
  ATTN_F32 = 1   /* q, kv_cache and out are float32 */
} attn_dtype;

/*
 * Host-side scalars describing one call. They mirror the scalar fields of the
 * FlashAttentionMetadata section of [FA] (num_actual_tokens, max_query_len, max_seq_len)
 * plus the per-layer constants of its FlashAttentionImpl section. Passing them from the
 * host keeps the call free of device-to-host synchronisation.
 */
typedef struct attn_desc {
  int32_t num_seqs;           /* requests in the batch */
  int32_t num_tokens;         /* query rows = query_start_loc[num_seqs] */
  int32_t num_decodes;        /* requests [0, num_decodes) have query_len == 1 ([LIN]) and
                                 take the split-KV decode path; 0 sends every request
                                 through the prefill kernel */
  int32_t max_query_len;      /* >= every query_len */
  int32_t max_seq_len;        /* >= every seq_len */
  int32_t num_heads;          /* query heads Hq */
  int32_t num_kv_heads;       /* Hkv; Hq % Hkv == 0; q head h reads kv head h / (Hq/Hkv) */
  int32_t head_size;          /* d: 64 or 128 */
  int32_t num_blocks;         /* physical blocks in kv_cache */
  int32_t block_size;         /* tokens per block, a positive multiple of 16 */
  int32_t max_blocks_per_seq; /* row stride of block_table */
  int32_t dtype;              /* attn_dtype */
  int32_t partition_tokens;   /* split-KV partition length for decode rows: a multiple of
                                 128 in [128, 16384], or 0 for the library's choice (the
                                 longest of 16384, 8192, ..., 256 that still yields 2048
                                 split workgroups for num_decodes requests of max_seq_len
                                 keys, else 256) */
} attn_desc;

/*
 * attn_workspace_bytes: device workspace that attn_varlen_fwd needs for `desc`.
 * It holds the per-partition partial outputs (normalised, bf16) and log-sum-exps (fp32) of
 * the decode rows ([RBLN] Overview: partition results combined by online softmax):
 *   num_decodes * num_heads * P * (head_size * 2 + 4) bytes, rounded up to 256,
 * where P is the number of partitions of max_seq_len (capped for a window in
 * attn_varlen_fwd), followed by the decode work schedule the call builds there:
 *   (1 + num_decodes * P) * 4 bytes, rounded up to 256.
 * A workspace serves one call at a time (calls that share one must not overlap).
 * Returns 0 bytes when num_decodes == 0 or dtype is ATTN_F32.
 * Errors: ATTN_ERR_NULL (desc or bytes NULL), and the same shape checks as attn_varlen_fwd
 * that do not depend on the window.
 */
attn_status attn_workspace_bytes(const attn_desc* desc, size_t* bytes);

/*
 * attn_decode_partition_tokens: the split-KV partition length (keys) that attn_varlen_fwd uses
 * for the decode rows of `desc`: desc->partition_tokens when it is set, else the library's
 * choice described at attn_desc.partition_tokens. A host-side query; nothing touches the GPU.
 * Errors: ATTN_ERR_NULL (desc or tokens NULL) and the descriptor errors of attn_workspace_bytes.
 */
attn_status attn_decode_partition_tokens(const attn_desc* desc, int32_t* tokens);

/*
 * attn_varlen_fwd: exact attention for a variable-length batch over a paged KV cache.
 *
 * For request r, let q0 = query_start_loc[r], ql = query_start_loc[r+1] - q0,
 * sl = seq_lens[r] and cl = sl - ql ([OTH] Triton section). Query row i (0 <= i < ql) sits at
 * absolute position p = cl + i. For every q head h, with kv head kh = h / (Hq/Hkv), it attends
 * to keys j in [0, sl) with j <= p when `causal` ([RBLN] Full Attention) and j >= p - window + 1
 * when window > 0 ([RBLN] SWA); key j is K/V row
 *   kv_cache[0 or 1][block_table[r * max_blocks_per_seq + j / block_size]][j % block_size][kh]
 * ([FA] Backend). With s_j = scale * q . k_j:
 *   out[q0+i][h] = sum_j softmax(s)_j v_j,   lse[q0+i][h] = ln sum_j exp(s_j).
 * A row with no visible key gets out = 0 and lse = -inf.
 *
 * Arguments (device pointers unless noted):
 *   desc            host pointer, see attn_desc.
 *   q               [num_tokens][num_heads][head_size], dtype of desc, rows packed by request.
 *   kv_cache        [2][num_blocks][block_size][num_kv_heads][head_size], dtype of desc.
 *                   Slots past seq_len and unused blocks are never read into the result.
 *   block_table     int32 [num_seqs][max_blocks_per_seq]; entries past a request's last
 *                   block are never read.
 *   query_start_loc int32 [num_seqs + 1], non-decreasing, query_start_loc[0] = 0.
 *   seq_lens        int32 [num_seqs], seq_len >= query_len.
 *   scale           softmax scale applied to q . k ([FA] Impl).
 *   causal          nonzero for causal masking (bottom-right aligned as above).
 *   window          > 0: sliding window of `window` keys including the query's own position;
 *                   requires causal. <= 0: no window.
 *   out             [num_tokens][num_heads][head_size], dtype of desc; every row is written.
 *   lse             float32 [num_tokens][num_heads], or NULL to skip it.
 *   workspace       device scratch of at least attn_workspace_bytes(desc) bytes (may be NULL
 *                   when that is 0); its contents on entry do not matter.
 *   workspace_bytes size of workspace.
 *   stream          hipStream_t to queue on (NULL = the null stream). The call returns as
 *                   soon as the kernels are queued.
 *
 * Errors: ATTN_ERR_NULL, ATTN_ERR_SHAPE (negative or inconsistent sizes, more than 65535
 * requests, than 65535 256-row query tiles of max_query_len or than 65535 decode partitions
 * of max_seq_len), ATTN_ERR_BLOCK_SIZE ([FA] Backend
 * raises on block_size % 16 != 0), ATTN_ERR_GQA, ATTN_ERR_UNSUPPORTED (head_size not 64/128, unknown
 * dtype, partition_tokens not a multiple of 128 in [128, 16384], window > 0 without
 * causal, scale not finite and > 0),
 * ATTN_ERR_WORKSPACE, ATTN_ERR_HIP (launch failure).
 */
attn_status attn_varlen_fwd(const attn_desc* desc, const void* q, const void* kv_cache,
                            const int32_t* block_table, const int32_t* query_start_loc,
                            const int32_t* seq_lens, float scale, int32_t causal,
                            int32_t window, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * attn_varlen_fwd_noalloc: attn_varlen_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation). It
 * takes no workspace: the decode rows' partial results and work schedule go to a fixed device
 * array of ATTN_NOALLOC_SCRATCH_BYTES bytes inside the library, of which every GPU the library
 * runs on holds one copy until the process ends (its address is looked up on the first call
 * on each device, with that device current; the caller's current device must be the one its
 * stream and tensors live on). The call allocates and frees nothing and runs the same kernels
 * as attn_varlen_fwd, so its results are identical.
 *
 * Every call on one GPU shares that GPU's array: calls that may overlap on one GPU (on
 * different streams, or from different threads without ordering) race on it and must not be
 * issued. Nothing in the array needs to start at zero; it keeps whatever the last call left.
 *
 * Arguments and errors: those of attn_varlen_fwd without workspace / workspace_bytes, plus
 * ATTN_ERR_WORKSPACE when the call would need more than ATTN_NOALLOC_SCRATCH_BYTES (i.e. when
 * attn_workspace_bytes, with the window's partition cap, exceeds it), and ATTN_ERR_HIP when the
 * array's device address cannot be obtained.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
attn_status attn_varlen_fwd_noalloc(const attn_desc* desc, const void* q, const void* kv_cache,
                                    const int32_t* block_table,
                                    const int32_t* query_start_loc, const int32_t* seq_lens,
                                    float scale, int32_t causal, int32_t window, void* out,
                                    float* lse, void* stream);

/*
 * attn_check_metadata_host: validates host copies of the metadata against desc:
 * query_start_loc starts at 0, is non-decreasing and ends at num_tokens; 0 <= query_len <=
 * seq_len <= max_seq_len; query_len <= max_query_len; requests [0, num_decodes) have
 * query_len == 1; ceil(seq_len / block_size) <= max_blocks_per_seq; every block id a request
 * uses lies in [0, num_blocks). All pointers are host pointers; nothing touches the GPU.
 * Returns ATTN_OK, ATTN_ERR_METADATA, or the desc errors of attn_varlen_fwd.
 */
attn_status attn_check_metadata_host(const attn_desc* desc, const int32_t* block_table,
                                     const int32_t* query_start_loc, const int32_t* seq_lens);

/*
 * Cascade attention for a prefix shared by every request of the batch ([FA] "Cascade
 * Attention: 공통 프리픽스 최적화" section, and the use_cascade / common_prefix_len fields of
 * its FlashAttentionMetadata section). The result is the same exact attention as
 * attn_varlen_fwd with window = 0; it is computed as
 *   1. a prefix pass: one sequence whose queries are all num_tokens query rows and whose keys
 *      are the first common_prefix_len keys (read through block_table row 0), not causal,
 *      written as fp32 partial results to the workspace;
 *   2. a suffix pass: every request over its keys [common_prefix_len, seq_len), causal when
 *      `causal` is set, merged with the prefix result through the log-sum-exps ([RBLN]
 *      Overview: partial softmax results combined) - inside the prefill kernel for prefill
 *      rows, in the partition merge kernel for decode rows.
 * The prefix K/V are read once per kv head for the whole batch instead of once per request.
 *
 * Preconditions (trusted on the device; attn_check_cascade_host checks host copies):
 *   common_prefix_len is a multiple of block_size; the first common_prefix_len / block_size
 *   block-table entries are the same for every request; every request's context length
 *   seq_len - query_len is >= common_prefix_len (each query sits after the prefix).
 * common_prefix_len == 0 is a plain attn_varlen_fwd call (window 0).
 *
 * attn_cascade_workspace_bytes: bytes of device workspace attn_cascade_fwd needs:
 *   num_tokens * num_heads * (head_size + 1) * 4 bytes (each part rounded up to 256) for the
 *   prefix result, plus attn_workspace_bytes(desc) for the decode partitions;
 *   attn_workspace_bytes(desc) alone when common_prefix_len == 0.
 * attn_cascade_fwd: arguments as attn_varlen_fwd (no window), plus common_prefix_len.
 * Errors: those of attn_varlen_fwd; ATTN_ERR_UNSUPPORTED for a dtype other than ATTN_BF16;
 * ATTN_ERR_SHAPE when common_prefix_len is negative, not a multiple of block_size or larger
 * than max_seq_len; ATTN_ERR_WORKSPACE when workspace_bytes is below
 * attn_cascade_workspace_bytes.
 */
attn_status attn_cascade_workspace_bytes(const attn_desc* desc, int32_t common_prefix_len,
                                         size_t* bytes);
attn_status attn_cascade_fwd(const attn_desc* desc, const void* q, const void* kv_cache,
                             const int32_t* block_table, const int32_t* query_start_loc,
                             const int32_t* seq_lens, int32_t common_prefix_len, float scale,
                             int32_t causal, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * attn_check_cascade_host: attn_check_metadata_host plus the cascade preconditions above
 * (shared prefix blocks, every context length >= common_prefix_len), on host copies.
 * Returns ATTN_OK, ATTN_ERR_METADATA, or the descriptor errors of attn_cascade_fwd.
 */
attn_status attn_check_cascade_host(const attn_desc* desc, const int32_t* block_table,
                                    const int32_t* query_start_loc, const int32_t* seq_lens,
                                    int32_t common_prefix_len);

/*
 * attn_kv_cache_write: store the new tokens' K and V rows in the paged cache through
 * slot_mapping ([FA] FlashAttentionMetadata section: slot_mapping beside block_table;
 * "왜 이 설계인가" item 2: block_table and slot_mapping reach a non-contiguous cache; cache
 * shape from the FlashAttentionBackend section). This is the step before attention in a layer:
 * afterwards attn_varlen_fwd reads these tokens through block_table.
 *
 * For t in [0, desc->num_tokens) with s = slot_mapping[t] >= 0:
 *   kv_cache[0][s / block_size][s % block_size][h][x] = key  [t * key_row_stride + h * head_size + x]
 *   kv_cache[1][s / block_size][s % block_size][h][x] = value[t * value_row_stride + h * head_size + x]
 * for every kv head h and x < head_size. A negative slot marks a padding token and writes
 * nothing; a slot >= num_blocks * block_size is skipped as well (never written out of bounds).
 * Slots of one call must be distinct (attn_check_slot_mapping_host checks host copies).
 *
 * Arguments (device pointers unless noted):
 *   desc             host pointer; uses num_tokens (new tokens), num_kv_heads, head_size,
 *                    num_blocks, block_size and dtype (of key, value and kv_cache alike).
 *   key, value       token rows of num_kv_heads * head_size elements, key_row_stride /
 *                    value_row_stride elements apart (>= num_kv_heads * head_size; e.g. the K
 *                    and V columns of a packed QKV projection). Rows must start on 16-byte
 *                    boundaries.
 *   slot_mapping     int64 [num_tokens].
 *   kv_cache         [2][num_blocks][block_size][num_kv_heads][head_size], updated in place.
 *   stream           hipStream_t (NULL = the null stream); the call returns once queued.
 * Errors: ATTN_ERR_NULL, ATTN_ERR_SHAPE (negative sizes, row strides smaller than a row or
 * not 16-byte multiples, misaligned pointers, more than 2^39 chunks), ATTN_ERR_BLOCK_SIZE,
 * ATTN_ERR_UNSUPPORTED (head_size not 64/128, unknown dtype), ATTN_ERR_HIP.
 */
attn_status attn_kv_cache_write(const attn_desc* desc, const void* key, int64_t key_row_stride,
                                const void* value, int64_t value_row_stride,
                                const int64_t* slot_mapping, void* kv_cache, void* stream);

/*
 * FP8 KV cache (E4M3). The Triton Attention section of [OTH] names an FP8 KV cache and [RBLN]
 * states which of its modes support one; neither fixes the format or the scaling, so this
 * library reads it as: OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * subnormals, NaN = exponent and mantissa all ones, no infinity, largest magnitude 448), one
 * fp32 scale per tensor for K and one for V, a code c standing for value(c) * scale. The
 * cache has the usual shape [2][num_blocks][block_size][num_kv_heads][head_size], one byte per
 * element.
 *
 * attn_kv_cache_write_fp8: as attn_kv_cache_write, with bf16 key / value rows (desc->dtype
 * must be ATTN_BF16) stored as the code nearest to x / scale (quotient in fp32, ties to even,
 * magnitudes beyond 448 saturated to 448; a NaN input gives a NaN code). Errors: those of
 * attn_kv_cache_write; ATTN_ERR_UNSUPPORTED for another dtype or a scale that is not finite
 * and > 0.
 */
attn_status attn_kv_cache_write_fp8(const attn_desc* desc, const void* key,
                                    int64_t key_row_stride, const void* value,
                                    int64_t value_row_stride, const int64_t* slot_mapping,
                                    float k_scale, float v_scale, void* kv_cache, void* stream);

/*
 * attn_fp8_decode_fwd: attn_varlen_fwd for a batch of decode rows only (num_decodes ==
 * num_seqs, query_len 1 each) over an E4M3 cache: the same exact attention with K and V
 * dequantised (value(code) * k_scale, value(code) * v_scale). q and out are bf16 (desc->dtype
 * ATTN_BF16), lse fp32; the codes are converted to bf16 exactly (every E4M3 value is a bf16
 * value) and k_scale / v_scale are applied to the scores and the output in fp32. With
 * desc->partition_tokens 0 the split-KV partition is attn_decode_partition_tokens' length
 * capped at 1024 keys (E4M3 streams faster in the one-wave units of partitions up to 1024
 * keys); a non-zero partition_tokens is used as given. Workspace:
 * attn_fp8_decode_workspace_bytes(desc), which is at least attn_workspace_bytes(desc).
 * Errors: those of attn_varlen_fwd; ATTN_ERR_UNSUPPORTED for num_decodes != num_seqs, a
 * dtype other than ATTN_BF16, or scales that are not finite and > 0.
 */
/*
 * attn_fp8_decode_workspace_bytes: device workspace bytes that attn_fp8_decode_fwd needs for
 * this descriptor (its partition as stated there), written to *bytes. Errors: ATTN_ERR_NULL
 * (bytes null) and the descriptor errors of attn_workspace_bytes.
 */
attn_status attn_fp8_decode_workspace_bytes(const attn_desc* desc, size_t* bytes);

attn_status attn_fp8_decode_fwd(const attn_desc* desc, const void* q, const void* kv_cache,
                                const int32_t* block_table, const int32_t* query_start_loc,
                                const int32_t* seq_lens, float scale, float k_scale,
                                float v_scale, int32_t window, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_check_slot_mapping_host: every slot of the host array slot_mapping[num_tokens] is
 * negative (padding) or below num_blocks * block_size, and the non-negative slots are
 * distinct. Returns ATTN_OK, ATTN_ERR_METADATA, ATTN_ERR_NULL, ATTN_ERR_SHAPE or
 * ATTN_ERR_BLOCK_SIZE.
 */
attn_status attn_check_slot_mapping_host(const attn_desc* desc, const int64_t* slot_mapping);

/*
 * Prefill work schedule built ahead of the attention call ([FA] FA3 section: the work
 * distribution is computed before the kernel and kept in a preallocated int32 buffer, so that
 * the launch is the same under graph capture). The schedule lists the batch's prefill work
 * items - (request, 256-row query tile) for requests [num_decodes, num_seqs) - sorted by the
 * number of 64-key tiles each must read (given causal / window), longest first; the scheduled
 * call dispatches its prefill workgroups in that order across the whole batch and launches
 * none for tiles past a request's last query row. A schedule depends only on
 * query_start_loc, seq_lens, causal and window, so one build serves every layer of a batch.
 *
 * attn_schedule_bytes: bytes of the schedule buffer: 4 * (1 + (num_seqs - num_decodes) *
 *   ceil(max_query_len / 256)), rounded up to 256. Errors: ATTN_ERR_NULL and the descriptor
 *   errors of attn_varlen_fwd; ATTN_ERR_SHAPE when the scheduled grid would exceed 2^31
 *   workgroups.
 * attn_build_schedule: queue the device kernel that writes the schedule (int32; element 0 is
 *   the item count, then the items) for the device metadata query_start_loc / seq_lens.
 *   Errors: those of attn_schedule_bytes; ATTN_ERR_WORKSPACE when schedule is NULL or
 *   schedule_bytes too small; ATTN_ERR_UNSUPPORTED for window > 0 without causal.
 * attn_varlen_fwd_scheduled: attn_varlen_fwd (bf16 only) whose prefill rows follow a schedule
 *   built for the same descriptor, metadata, causal and window (not checked: it would need a
 *   device-to-host synchronisation). The results are identical to attn_varlen_fwd's.
 */
attn_status attn_schedule_bytes(const attn_desc* desc, size_t* bytes);
attn_status attn_build_schedule(const attn_desc* desc, const int32_t* query_start_loc,
                                const int32_t* seq_lens, int32_t causal, int32_t window,
                                int32_t* schedule, size_t schedule_bytes, void* stream);
attn_status attn_varlen_fwd_scheduled(const attn_desc* desc, const void* q, const void* kv_cache,
                                      const int32_t* block_table,
                                      const int32_t* query_start_loc, const int32_t* seq_lens,
                                      float scale, int32_t causal, int32_t window, void* out,
                                      float* lse, void* workspace, size_t workspace_bytes,
                                      const int32_t* schedule, size_t schedule_bytes,
                                      void* stream);

/*
 * Decode work schedule built ahead of the attention call (the same [FA] FA3 reasoning as the
 * prefill schedule above, applied to the split-KV decode rows whose partitions [RBLN] Overview
 * combines by online softmax). attn_varlen_fwd builds this schedule in its workspace on every
 * call with one small kernel: the (decode request, segment) items that hold visible keys,
 * sorted by the number of keys each reads, longest first. A segment is one partition, or, for
 * partitions of at most 1024 keys, floor(1024 / partition_tokens) consecutive partitions (one
 * wave streams them and writes one partial result per partition). The schedule depends only
 * on seq_lens, the window and the partition length, so a batch builds it once and every layer
 * reuses it.
 *
 * attn_decode_schedule_bytes: bytes of the decode schedule buffer for `window`: the schedule
 *   region of attn_workspace_bytes with P capped for the window (room for one item per
 *   partition, at least one per segment); 0 when the call has no
 *   split-KV decode rows (num_decodes == 0 or dtype ATTN_F32). Errors: ATTN_ERR_NULL and the
 *   descriptor errors of attn_workspace_bytes.
 * attn_build_decode_schedule: queue the kernel that writes the decode schedule (int32; element
 *   0 is the item count, then the items) for the device array seq_lens. Does nothing when attn_decode_schedule_bytes gives 0. Errors: those of
 *   attn_decode_schedule_bytes; ATTN_ERR_WORKSPACE when schedule is NULL or schedule_bytes
 *   too small; ATTN_ERR_NULL for a NULL seq_lens.
 * attn_varlen_fwd_prescheduled: attn_varlen_fwd that reads either schedule from the caller
 *   instead of building it: prefill_schedule (bf16 only) from attn_build_schedule,
 *   decode_schedule from attn_build_decode_schedule, each built for the same descriptor,
 *   metadata, causal and window (not checked: it would need a device-to-host
 *   synchronisation). Either may be NULL: that part is then scheduled as in attn_varlen_fwd.
 *   A schedule is only read, so calls on any streams may share it. The workspace is still
 *   attn_workspace_bytes(desc) (the decode partials live there). The results are identical
 *   to attn_varlen_fwd's. Errors: those of attn_varlen_fwd, plus ATTN_ERR_WORKSPACE for a
 *   schedule buffer below its size and ATTN_ERR_UNSUPPORTED for a prefill schedule with a
 *   dtype other than ATTN_BF16.
 */
attn_status attn_decode_schedule_bytes(const attn_desc* desc, int32_t window, size_t* bytes);
attn_status attn_build_decode_schedule(const attn_desc* desc, const int32_t* seq_lens,
                                       int32_t window, int32_t* schedule,
                                       size_t schedule_bytes, void* stream);
attn_status attn_varlen_fwd_prescheduled(
    const attn_desc* desc, const void* q, const void* kv_cache, const int32_t* block_table,
    const int32_t* query_start_loc, const int32_t* seq_lens, float scale, int32_t causal,
    int32_t window, void* out, float* lse, void* workspace, size_t workspace_bytes,
    const int32_t* prefill_schedule, size_t prefill_schedule_bytes,
    const int32_t* decode_schedule, size_t decode_schedule_bytes, void* stream);

/*
 * attn_varlen_fwd_mixed: attn_varlen_fwd (bf16 only) as ONE kernel launch for a batch that mixes
 * decode and prefill rows ([FA] "FA3의 AOT 스케줄링" section: one kernel serving mixed
 * prefill + decode batches; [LIN] Prefill/Decode split section: requests [0, num_decodes) are
 * the decode rows). Its first workgroups take the decode rows, one wave per (decode request, kv
 * head, group of up to 16 q heads) streaming all of the request's visible keys with an online
 * softmax and writing the output directly (no split-KV partitions, so no merge and no
 * workspace); the other workgroups are the prefill kernel's, taking their (request, q tile)
 * items from prefill_schedule (attn_build_schedule for the same descriptor, metadata, causal and
 * window). Same inputs, outputs and masks as attn_varlen_fwd; the decode rows' results equal
 * attn_varlen_fwd's up to the order of the fp32 softmax sums (one partition per request).
 * Errors: those of attn_varlen_fwd except the workspace ones; ATTN_ERR_UNSUPPORTED for a dtype
 * other than ATTN_BF16; ATTN_ERR_WORKSPACE when prefill rows exist and prefill_schedule is NULL
 * or below attn_schedule_bytes(desc).
 */
attn_status attn_varlen_fwd_mixed(const attn_desc* desc, const void* q, const void* kv_cache,
                                  const int32_t* block_table, const int32_t* query_start_loc,
                                  const int32_t* seq_lens, float scale, int32_t causal,
                                  int32_t window, void* out, float* lse,
                                  const int32_t* prefill_schedule, size_t prefill_schedule_bytes,
                                  void* stream);

/* attn_status_str: static, NUL-terminated name of a status code ("ATTN_OK", ...). */
const char* attn_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
