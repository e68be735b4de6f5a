// Device-side work schedule of the prefill kernel, for gfx950.
//
// The FA3 section of the "[vLLM] FlashAttention" page describes scheduling metadata that is
// computed before the attention kernel runs and kept in a preallocated int32 buffer, so that
// the work distribution is known ahead of the launch (and survives graph capture). This is
// that idea for this library's prefill kernel: one workgroup lists the batch's work items -
// (prefill request, 256-row query tile) - and counting-sorts them by their number of 64-key
// tiles, longest first. The prefill kernel then takes item i from the list (times the q heads),
// so the hardware's in-order workgroup dispatch hands out the heaviest tiles of the whole batch
// first and no workgroup is launched for a tile past a request's last query row.
//
// Schedule buffer (int32): [0] = number of items n, [1 + i] = item i (i < n) as
// request_offset * max_qtiles + q_tile, request_offset counting from the first prefill request.
//
// The split-KV decode kernel gets the same treatment: its items are (decode request,
// partition) pairs, sorted by their number of keys, so that the partial last partitions of the
// requests run at the end of the grid instead of being spread over it.
#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kSchedThreads = 1024;
constexpr int kBuckets = 4096;          // costs >= kBuckets - 1 share the top bucket

__device__ __forceinline__ int item_cost(const ScheduleParams& p, int e) {
  const int r = p.seq_begin + e / p.max_qtiles;
  const int qt = e % p.max_qtiles;
  const int q0 = p.qsl[r];
  const int ql = p.qsl[r + 1] - q0;
  if (qt * 256 >= ql) return -1;                              // past the last query row
  const int sl = p.seq_lens[r];
  const int cl = sl - ql;
  const int row_lo = qt * 256;
  const int row_hi = min(ql, row_lo + 256) - 1;
  const int kv_hi = p.causal ? min(sl, cl + row_hi + 1) : sl;
  const int kv_lo = p.window > 0 ? max(0, cl + row_lo - p.window + 1) : 0;
  const int tiles = (kv_hi + 63) / 64 - kv_lo / 64;
  return max(tiles, 0);
}

// Counting sort of the items [0, n_all) by cost, longest first, into schedule (one workgroup
// of kSchedThreads threads); cost(e) < 0 drops item e. Items of equal cost keep no fixed order.
template <class Cost>
__device__ void sort_items(int n_all, Cost cost, int32_t* schedule) {
  __shared__ int hist[kBuckets];
  const int tid = threadIdx.x;
  for (int b = tid; b < kBuckets; b += kSchedThreads) hist[b] = 0;
  __syncthreads();
  // 1. histogram of the costs (bucket kBuckets - 1 - cost, so that bucket order is longest first)
  for (int e = tid; e < n_all; e += kSchedThreads) {
    const int c = cost(e);
    if (c >= 0) atomicAdd(&hist[kBuckets - 1 - min(c, kBuckets - 1)], 1);
  }
  __syncthreads();
  // 2. exclusive prefix sum over the buckets: each thread scans 4 buckets, then the 1024
  //    partial sums are scanned by one wave-serial pass in LDS
  __shared__ int part[kSchedThreads];
  constexpr int per = kBuckets / kSchedThreads;
  int local[per];
  int s = 0;
#pragma unroll
  for (int k = 0; k < per; ++k) {
    local[k] = s;
    s += hist[tid * per + k];
  }
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < kSchedThreads; off <<= 1) {   // Hillis-Steele inclusive scan
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  const int base = tid > 0 ? part[tid - 1] : 0;
#pragma unroll
  for (int k = 0; k < per; ++k) hist[tid * per + k] = base + local[k];   // bucket start
  const int total = part[kSchedThreads - 1];
  __syncthreads();
  // 3. scatter the items to their sorted positions
  for (int e = tid; e < n_all; e += kSchedThreads) {
    const int c = cost(e);
    if (c < 0) continue;
    const int pos = atomicAdd(&hist[kBuckets - 1 - min(c, kBuckets - 1)], 1);
    schedule[1 + pos] = e;
  }
  if (tid == 0) schedule[0] = total;
}

__global__ __launch_bounds__(kSchedThreads) void prefill_schedule_kernel(const ScheduleParams p) {
  sort_items(p.num_seqs * p.max_qtiles, [&](int e) { return item_cost(p, e); }, p.schedule);
}

// Keys of partition pi of decode request r (the partition split of the decode kernel), in
// 16-key units; -1 past the request's last partition.
__device__ __forceinline__ int decode_item_cost(const DecodeScheduleParams& p, int e) {
  const int r = e / p.max_parts;
  const int pi = e % p.max_parts;
  const int sl = p.seq_lens[r] - p.kv_skip_keys;
  int first, nparts;
  decode_partitions(sl, p.window, p.part_tokens, &first, &nparts);
  if (pi >= min(nparts, p.max_parts)) return -1;
  const int lo = p.window > 0 ? max(0, sl - p.window) : 0;
  const int part = first + pi;
  const int keys = min(sl, (part + 1) * p.part_tokens) - max(lo, part * p.part_tokens);
  return (keys + 15) / 16;
}

__global__ __launch_bounds__(kSchedThreads) void decode_schedule_kernel(
    const DecodeScheduleParams p) {
  sort_items(p.num_decodes * p.max_parts, [&](int e) { return decode_item_cost(p, e); },
             p.schedule);
}

}  // namespace

hipError_t launch_decode_schedule(const DecodeScheduleParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(decode_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_prefill_schedule(const ScheduleParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(prefill_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
