// Split-KV decode attention (query_len == 1) and the log-sum-exp merge, bf16, for gfx950.
//
// Method: the RBLN "Attention 모드" page (Overview, Flash Attention bullet) processes each
// request's KV cache partition by partition and combines the per-partition results with online
// softmax. Here one unit of work is one (decode request, kv head, partition of part_tokens
// keys) with all q heads that share that kv head (num_queries_per_kv of the vLLM
// FlashAttention page's FlashAttentionImpl section), so every K/V byte is read from HBM once
// per kv head. The partition result goes to the workspace - the normalised output rounded to
// bf16 (a convex combination of V rows, so the rounding adds at most 2^-9 of its magnitude,
// as the bf16 output itself does; writing fp32 there cost ~8 % of the decode time at 512-key
// partitions, writes being dear in a read-saturated stream) and its log-sum-exp in fp32 - and
// a second kernel merges the partitions of each (request, q head) through their log-sum-exp
// in fp32. A request whose visible keys fit one partition is written directly.
//
// A unit runs on one wave (partitions of up to 1024 keys) or on a 4-wave workgroup whose
// waves take a quarter of the partition each and combine through LDS (longer partitions).
// A wave streams its keys in 32-key chunks, two chunks' loads in flight ahead of the math:
//   * S^T = K . Q^T on v_mfma_f32_16x16x32_bf16, the q heads of the group in the 16 MFMA
//     columns;
//   * V rows are copied into a wave-private LDS tile and read back transposed with
//     ds_read_b64_tr_b16 as the A operand of O^T += V^T . P^T.
#include <type_traits>

#include "decode_core.hpp"
#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

using namespace dec;

constexpr int kWaves = 4;

// The decode work item in schedule slot `slot` for (kv head, head group) `hw`, and the keys it
// reads. valid is false for slots past the item count.
struct DecodeItem {
  bool valid;
  int r, hw, kvh, nh, h0, tok;
  int first_part, nparts;        // the request's partitions holding visible keys
  int p_start, k_begin, k_end;   // segment start, its visible keys [k_begin, k_end)
};
__device__ __forceinline__ DecodeItem decode_item(const DecodeParams& p, int slot, int hw) {
  DecodeItem it{};
  const int group = p.num_heads / p.num_kv_heads;
  const int head_groups = (group + 15) / 16;
  const int count = p.items[0];
  const int item = p.items[1 + min(slot, p.num_decodes * p.max_segs - 1)];
  it.valid = slot < count;
  if (!it.valid) return it;
  it.r = item / p.max_segs;
  const int si = item % p.max_segs;
  it.hw = hw;
  it.kvh = hw / head_groups;
  const int hg = hw % head_groups;
  it.nh = min(16, group - hg * 16);                   // q heads of this unit
  it.h0 = it.kvh * group + hg * 16;                   // first q head
  // keys of this pass: [0, sl) after skipping kv_skip_blocks leading blocks
  const int sl = p.seq_lens[it.r] - p.kv_skip_blocks * p.block_size;
  int first_seg, nsegs;
  decode_partitions(sl, p.window, p.seg_tokens, &first_seg, &nsegs);
  decode_partitions(sl, p.window, p.part_tokens, &it.first_part, &it.nparts);
  it.nparts = min(it.nparts, p.max_parts);   // only reachable with seq_len > max_seq_len
  it.p_start = (first_seg + si) * p.seg_tokens;
  const int lo = p.window > 0 ? max(0, sl - p.window) : 0;
  it.k_begin = max(lo, it.p_start);
  it.k_end = min(sl, it.p_start + p.seg_tokens);
  it.tok = p.qsl[it.r];
  return it;
}

// FP8 = true: the cache holds E4M3 codes (one byte per element) with per-tensor scales; the
// host folds k_scale into p.scale and the kernel multiplies the output by p.v_scale.
//
// Workgroup mode (partitions of more than kWaveSegmentTokens keys, one per segment): one
// workgroup of 4 waves per (item, kv head, head group); each wave streams its own quarter of
// the partition and the 4 waves' (max, sum, O) are combined through LDS at the end.
template <int D, bool FP8>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(const DecodeParams p) {
  using T = WaveTiles<D>;
  constexpr int OS = D + 4;            // fp32 row stride of the combine buffer
  // V tiles during the stream; reused as the combine buffer afterwards
  constexpr int kLdsBytes = (kWaves * T::V_TILE * 2 > kWaves * 16 * OS * 4)
                                ? kWaves * T::V_TILE * 2 : kWaves * 16 * OS * 4;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
  __shared__ float sM[kWaves][16];
  __shared__ float sL[kWaves][16];
  __shared__ int32_t sBlk[kMaxPartitionTokens / 16];   // block ids of this partition
  __shared__ __attribute__((aligned(16))) __bf16 sK[FP8 ? 8 : kWaves * T::K_TILE];

  // grid x = item slot * heads_wg + (kv head, head group): the workgroups of one item read
  // the same tokens' rows (adjacent in every cache block) side by side, and the items come
  // from the decode schedule, longest partition first
  const int heads_wg = p.num_kv_heads * ((p.num_heads / p.num_kv_heads + 15) / 16);
  const DecodeItem it = decode_item(p, blockIdx.x / heads_wg, blockIdx.x % heads_wg);
  if (!it.valid) return;

  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int lane = tid % kWave;
  const int G = lane / 16;
  const int li = lane % 16;

  // block ids covering [p_start, k_end) -> LDS, so the K/V loads need no dependent lookup
  const int b_first = it.p_start / p.block_size;
  const int n_blk = (it.k_end - 1) / p.block_size - b_first + 1;
  const int32_t* __restrict__ bt =
      p.block_table + (int64_t)it.r * p.max_blocks + p.kv_skip_blocks;
  for (int i = tid; i < n_blk; i += 256) sBlk[i] = bt[b_first + i];

  bf16x8 qf[D / 32];
  load_q_frag<D, FP8>(p, it.tok, it.h0, it.nh, qf);

  // this wave's key range: quarter w of the partition, clipped to the visible range; chunks
  // are aligned to the quarter start (a multiple of 32)
  const int quarter = p.part_tokens / kWaves;
  const int c_base = it.p_start + w * quarter;
  const int w_begin = max(it.k_begin, c_base);
  const int w_end = min(it.k_end, c_base + quarter);
  __bf16* sVw = reinterpret_cast<__bf16*>(lds) + w * T::V_TILE;
  __bf16* sKw = sK + (FP8 ? 0 : w * T::K_TILE);
  __syncthreads();   // sBlk ready

  float m_run, l_run;
  floatx4 o[D / 16];
  init_state(m_run, l_run, o, D / 16);
  stream_keys<D, FP8>(p, it.kvh, qf, c_base, w_begin, w_end, it.k_end - 1,
                      [&](uint32_t bidx) __attribute__((always_inline)) {
                        return sBlk[bidx - b_first];
                      },
                      sVw, sKw, m_run, l_run, o, [](int) {});

  // ---- combine the 4 waves: (m, l, O^T) -> partition result
  const float c_log2 = p.scale * kLog2e;
  const float l_w = column_sum(l_run);
  __syncthreads();   // every wave is done with its V tile; the LDS becomes the combine buffer
  float* sO = reinterpret_cast<float*>(lds);
  if (G == 0) {
    sM[w][li] = m_run;
    sL[w][li] = l_w;
  }
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc)
    *reinterpret_cast<floatx4*>(&sO[(w * 16 + li) * OS + 16 * dc + 4 * G]) = o[dc];
  __syncthreads();

  constexpr int DPT = D / 16;          // d values per thread: 256 threads = 16 heads x 16
  const int hh = tid / 16;             // head within the workgroup
  const int d0 = (tid % 16) * DPT;
  if (hh >= it.nh) return;
  float M = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sM[ww][hh]);
  const float M_use = (M == -INFINITY) ? 0.f : M;
  float wgt[kWaves];
  float L = 0.f;
#pragma unroll
  for (int ww = 0; ww < kWaves; ++ww) {
    wgt[ww] = fast_exp2((sM[ww][hh] - M_use) * c_log2);
    L += sL[ww][hh] * wgt[ww];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float acc[DPT];
#pragma unroll
  for (int x = 0; x < DPT; ++x) {
    float a = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) a += wgt[ww] * sO[(ww * 16 + hh) * OS + d0 + x];
    acc[x] = FP8 ? a * inv * p.v_scale : a * inv;
  }
  const float lse_part = L > 0.f ? p.scale * M + __logf(L) : -INFINITY;
  const int hq = it.h0 + hh;
  if (it.nparts == 1 && p.pre_o == nullptr) {
    __bf16* dst = static_cast<__bf16*>(p.out) + ((int64_t)it.tok * p.num_heads + hq) * D + d0;
#pragma unroll
    for (int x = 0; x < DPT; ++x) dst[x] = to_bf16(acc[x]);
    if (p.lse != nullptr && d0 == 0) p.lse[(int64_t)it.tok * p.num_heads + hq] = lse_part;
  } else {
    const int pi = it.k_begin / p.part_tokens - it.first_part;   // the segment's partition
    const int64_t slot = ((int64_t)it.r * p.num_heads + hq) * p.max_parts + pi;
    __bf16* dst = p.ws_o + slot * D + d0;
#pragma unroll
    for (int x = 0; x < DPT; ++x) dst[x] = to_bf16(acc[x]);
    if (d0 == 0) p.ws_lse[slot] = lse_part;
  }
}

// Wave mode (partitions of at most kWaveSegmentTokens keys): each wave of a 4-wave workgroup
// is one (item, kv head, head group) unit and streams the item's whole segment alone (no
// cross-wave combine, no barrier), writing one result per partition of the segment as its
// last chunk is consumed: a segment of several short partitions pays the unit's start-up
// (schedule slot, block ids, Q^T, the first loads) once. The segment's block ids (at most 64)
// sit one per lane and reach the address computation through v_readlane. Units are numbered
// like the workgroup mode's grid (item slot * heads_wg + (kv head, head group)), 4 consecutive
// units per workgroup.
template <int D, bool FP8>
__global__ __launch_bounds__(256, 2) void decode_wave_kernel(const DecodeParams p) {
  using T = WaveTiles<D>;
  __shared__ __attribute__((aligned(16))) __bf16 sV[kWaves * T::V_TILE];
  __shared__ __attribute__((aligned(16))) __bf16 sK[FP8 ? 8 : kWaves * T::K_TILE];

  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int G = lane / 16;
  const int li = lane % 16;
  const int heads_wg = p.num_kv_heads * ((p.num_heads / p.num_kv_heads + 15) / 16);
  const int unit = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + w);
  const DecodeItem it = decode_item(p, unit / heads_wg, unit % heads_wg);
  if (!it.valid) return;

  // lane i holds the cache block of the segment's i-th block (n_blk <= 64: the segment has at
  // most kWaveSegmentTokens keys and block_size is a multiple of 16)
  const int b_first = it.p_start / p.block_size;
  const int n_blk = (it.k_end - 1) / p.block_size - b_first + 1;
  const int32_t* __restrict__ bt =
      p.block_table + (int64_t)it.r * p.max_blocks + p.kv_skip_blocks;
  const int32_t blk_lane = lane < n_blk ? bt[b_first + lane] : 0;

  bf16x8 qf[D / 32];
  load_q_frag<D, FP8>(p, it.tok, it.h0, it.nh, qf);

  float m_run, l_run;
  floatx4 o[D / 16];
  init_state(m_run, l_run, o, D / 16);
  // after the chunk at key kb: at the end of a partition (or of the segment), its result
  // goes out (lane (G, li) holds O^T rows d = 16 dc + 4 G .. +3 of q head h0 + li) and the
  // state restarts for the next partition
  auto after = [&](int kb) __attribute__((always_inline)) {
    const int k_next = kb + kChunk;
    if (k_next % p.part_tokens != 0 && k_next < it.k_end) return;
    const int pi = kb / p.part_tokens - it.first_part;
    const float l = column_sum(l_run);
    const float inv = l > 0.f ? (FP8 ? p.v_scale : 1.f) / l : 0.f;
    const float lse_part = l > 0.f ? p.scale * m_run + __logf(l) : -INFINITY;
    const int hq = it.h0 + li;
    if (li < it.nh) {
      if (it.nparts == 1 && p.pre_o == nullptr) {
        __bf16* dst = static_cast<__bf16*>(p.out) + ((int64_t)it.tok * p.num_heads + hq) * D;
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) {
          const floatx4 v = o[dc] * inv;
          bf16x4 b4;
#pragma unroll
          for (int e = 0; e < 4; ++e) b4[e] = to_bf16(v[e]);
          *reinterpret_cast<bf16x4*>(dst + 16 * dc + 4 * G) = b4;
        }
        if (p.lse != nullptr && G == 0) p.lse[(int64_t)it.tok * p.num_heads + hq] = lse_part;
      } else if (pi < p.max_parts) {   // only false with seq_len > max_seq_len
        const int64_t slot = ((int64_t)it.r * p.num_heads + hq) * p.max_parts + pi;
        __bf16* dst = p.ws_o + slot * D;
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) {
          const floatx4 v = o[dc] * inv;
          bf16x4 b4;
#pragma unroll
          for (int e = 0; e < 4; ++e) b4[e] = to_bf16(v[e]);
          *reinterpret_cast<bf16x4*>(dst + 16 * dc + 4 * G) = b4;
        }
        if (G == 0) p.ws_lse[slot] = lse_part;
      }
    }
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) o[dc] = floatx4{0.f, 0.f, 0.f, 0.f};
  };
  stream_keys<D, FP8>(p, it.kvh, qf, it.p_start, it.k_begin, it.k_end, it.k_end - 1,
                      [&](uint32_t bidx) __attribute__((always_inline)) {
                        return __builtin_amdgcn_readlane(blk_lane, (int)(bidx - b_first));
                      },
                      sV + w * T::V_TILE, sK + (FP8 ? 0 : w * T::K_TILE), m_run, l_run, o,
                      after);
}

// One wave per (q head, decode request): out = sum_p exp(lse_p - L) o_p and lse = L =
// log sum_p exp(lse_p) over the request's partitions plus, in a cascade suffix pass, the
// prefix's partial result. The partitions are read kMergeBatch at a time with all their loads
// in flight together, and folded into a running (max, sum, weighted output), so a merge takes
// one memory round trip per kMergeBatch partitions.
constexpr int kMergeBatch = 16;
template <int D>
__global__ __launch_bounds__(64) void lse_merge_kernel(const DecodeParams p) {
  const int hq = blockIdx.x;
  const int r = blockIdx.y;
  const int sl = p.seq_lens[r] - p.kv_skip_blocks * p.block_size;
  int first, nparts;
  decode_partitions(sl, p.window, p.part_tokens, &first, &nparts);
  nparts = min(nparts, p.max_parts);
  const bool pre = p.pre_o != nullptr;
  if (nparts <= 1 && !pre) return;        // written directly by the split kernel
  const int lane = threadIdx.x;
  const int tok = p.qsl[r];
  const int64_t base = ((int64_t)r * p.num_heads + hq) * p.max_parts;
  const int64_t row = (int64_t)tok * p.num_heads + hq;
  constexpr int DPL = D / kWave;
  float m = -INFINITY, s = 0.f;
  float acc[DPL];
#pragma unroll
  for (int x = 0; x < DPL; ++x) acc[x] = 0.f;
  if (pre) {
    const float lp = p.pre_lse[row];
    if (lp != -INFINITY) {
      m = lp;
      s = 1.f;
#pragma unroll
      for (int x = 0; x < DPL; ++x) acc[x] = p.pre_o[row * D + lane + kWave * x];
    }
  }
  for (int p0 = 0; p0 < nparts; p0 += kMergeBatch) {
    float l[kMergeBatch], v[kMergeBatch][DPL];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const int64_t slot = base + min(p0 + i, nparts - 1);   // past the end: masked below
      l[i] = p.ws_lse[slot];
#pragma unroll
      for (int x = 0; x < DPL; ++x) v[i][x] = (float)p.ws_o[slot * D + lane + kWave * x];
    }
    float mb = m;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i)
      if (p0 + i < nparts) mb = fmaxf(mb, l[i]);
    const float mu = (mb == -INFINITY) ? 0.f : mb;
    const float a = fast_exp2((m - mu) * kLog2e);          // 0 while nothing is merged
    s *= a;
#pragma unroll
    for (int x = 0; x < DPL; ++x) acc[x] *= a;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      if (p0 + i >= nparts) break;
      const float w = fast_exp2((l[i] - mu) * kLog2e);
      s += w;
#pragma unroll
      for (int x = 0; x < DPL; ++x) acc[x] += w * v[i][x];
    }
    m = mb;
  }
  const float inv = s > 0.f ? 1.f / s : 0.f;
  __bf16* dst = static_cast<__bf16*>(p.out) + row * D;
#pragma unroll
  for (int x = 0; x < DPL; ++x) dst[lane + kWave * x] = to_bf16(acc[x] * inv);
  if (p.lse != nullptr && lane == 0) p.lse[row] = s > 0.f ? m + __logf(s) : -INFINITY;
}

// The schedule kernel (unless the caller built the schedule ahead), then the split kernel
// (one wave or workgroup per (schedule slot, kv head, head group), slots past the item count
// exiting at once), then the merge.
template <int D, bool FP8>
hipError_t launch(const DecodeParams& p, hipStream_t stream) {
  const int head_groups = (p.num_heads / p.num_kv_heads + 15) / 16;
  DecodeParams pk = p;
  if (pk.items == nullptr) {
    DecodeScheduleParams sp{};
    sp.seq_lens = p.seq_lens;
    sp.schedule = p.schedule;
    sp.num_decodes = p.num_decodes;
    sp.part_tokens = p.seg_tokens;
    sp.max_parts = p.max_segs;
    sp.window = p.window;
    sp.kv_skip_keys = p.kv_skip_blocks * p.block_size;
    const hipError_t e = launch_decode_schedule(sp, stream);
    if (e != hipSuccess) return e;
    pk.items = p.schedule;
  }
  const int64_t units = (int64_t)p.num_decodes * p.max_segs * p.num_kv_heads * head_groups;
  if (p.part_tokens <= kWaveSegmentTokens)
    hipLaunchKernelGGL((decode_wave_kernel<D, FP8>), dim3((unsigned)((units + kWaves - 1) / kWaves)),
                       dim3(256), 0, stream, pk);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, FP8>), dim3((unsigned)units), dim3(256), 0,
                       stream, pk);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || (p.max_parts <= 1 && p.pre_o == nullptr)) return e;
  hipLaunchKernelGGL(lse_merge_kernel<D>, dim3(p.num_heads, p.num_decodes), dim3(kWave), 0,
                     stream, pk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeParams& p, hipStream_t stream) {
  if (p.num_decodes <= 0) return hipSuccess;
  return p.head_size == 64 ? launch<64, false>(p, stream) : launch<128, false>(p, stream);
}

hipError_t launch_decode_fp8(const DecodeParams& p, hipStream_t stream) {
  if (p.num_decodes <= 0) return hipSuccess;
  return p.head_size == 64 ? launch<64, true>(p, stream) : launch<128, true>(p, stream);
}

}  // namespace attn
