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

#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kChunk = 32;       // keys per wave iteration

// 8 E4M3 codes (two 32-bit words) -> 8 bf16 values, exactly (every E4M3 value is a bf16
// value; v_cvt_scalef32_pk_bf16_fp8 with scale 1 converts two codes, checked on gfx950 for all
// 256 codes).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Q^T (B operand of the QK^T product) for q heads h0 .. h0 + nh - 1 of token tok: lane
// (G, li) holds q head h0 + li at the d values its K operand holds: d = 32c + 8G .. +7 (bf16),
// or d = 64(c/2) + 16G + 8(c%2) .. +7 for E4M3 K, where lane G reads bytes 64w + 16G .. +15 of
// the row with load w, so that each load instruction covers 64 contiguous bytes of 16 rows
// (any fixed order of d is the same dot product). Lanes past nh hold zeros.
template <int D, bool FP8>
__device__ __forceinline__ void load_q_frag(const DecodeParams& p, int tok, int h0, int nh,
                                            bf16x8 (&qf)[D / 32]) {
  const int lane = threadIdx.x % kWave;
  const int G = lane / 16;
  const int li = lane % 16;
  const __bf16* __restrict__ q = static_cast<const __bf16*>(p.q);
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const int d0 = FP8 ? 64 * (c / 2) + 16 * G + 8 * (c % 2) : 32 * c + 8 * G;
    qf[c] = li < nh ? *reinterpret_cast<const bf16x8*>(
                          q + ((int64_t)tok * p.num_heads + h0 + li) * D + d0)
                    : bf16x8{};
  }
}

// LDS one wave uses while streaming: a V chunk tile (read back transposed) and, for bf16, a K
// chunk tile (bf16 elements each).
template <int D>
struct WaveTiles {
  static constexpr int RS = D + 16;            // row stride of a V chunk
  static constexpr int V_TILE = kChunk * RS;
  // bf16 K also goes through a wave-private LDS tile: its rows are loaded like V's (whole
  // 256-byte rows, 4 per instruction), which streams about 9 % faster on gfx950 than loading
  // the MFMA operand layout straight from HBM (16 rows x 64 bytes per instruction)
  static constexpr int KRS = D + 8;            // row stride of a K chunk
  static constexpr int K_TILE = kChunk * KRS;
};

// One wave's online-softmax pass over the keys [w_begin, w_end) of a decode request, for the
// q heads whose Q^T fragment is qf (kv head kvh), in 32-key chunks aligned to c_base (the
// chunk of w_begin is the first one). last_key is the request's last key in this partition:
// loads past it read that key's group again (clamped), so every load reads a valid row of the
// request; keys outside [w_begin, w_end) get score -inf. block_of(b) gives the cache block of
// the request's b-th block of this pass. Returns, per lane (G, li), the running max m_run and
// this lane's share of the running sum l_run (scores of column li; m_run is the same in
// every lane of a column), and O^T: o[dc][e] = sum_j p_j V[j][16 dc + 4 G + e] for q head
// li, unnormalised.
//   * S^T = K . Q^T on v_mfma_f32_16x16x32_bf16 (K rows in the A operand, q heads in the 16
//     columns);
//   * V rows are copied into the wave's LDS tile and read back transposed with
//     ds_read_b64_tr_b16 as the A operand of O^T += V^T . P^T.
template <int D, bool FP8, class BlockOf, class After>
__device__ __forceinline__ void stream_keys(const DecodeParams& p, int kvh,
                                            const bf16x8 (&qf)[D / 32], int c_base, int w_begin,
                                            int w_end, int last_key, BlockOf block_of,
                                            __bf16* sVw, __bf16* sKw, float& m_run,
                                            float& l_run, floatx4 (&o)[D / 16], After after) {
  using T = WaveTiles<D>;
  constexpr int RS = T::RS;
  constexpr int KRS = T::KRS;
  constexpr int KC = D / 32;
  constexpr int DC = D / 16;
  constexpr int EPL = FP8 ? 16 : 8;    // V elements per lane and copy instruction (16 bytes)
  constexpr int TPR = D / EPL;         // lanes per V row in the copy
  constexpr int RPI = kWave / TPR;     // V rows per copy instruction
  constexpr int NV = kChunk / RPI;     // copy instructions per chunk
  const int lane = threadIdx.x % kWave;
  const int G = lane / 16;
  const int li = lane % 16;
  const int v_row = lane / TPR;
  const int v_chunk = lane % TPR;

  const int c_first = w_end > w_begin ? (w_begin - c_base) / kChunk : 0;
  const int n_chunks =
      w_end > w_begin ? (w_end - (c_base + c_first * kChunk) + kChunk - 1) / kChunk : 0;

  typedef typename std::conditional<FP8, uint8_t, __bf16>::type kv_t;
  const kv_t* __restrict__ kcache = static_cast<const kv_t*>(p.kv);
  const kv_t* __restrict__ vcache = kcache + p.v_offset;

  // raw K / V of one chunk: bf16 K as whole rows like V (instruction j = k[j / KW][j % KW]),
  // E4M3 K as D/64 16-byte words per lane (word w at byte 64w + 16G); V as 16 bytes per lane and
  // instruction (8 bf16 or 16 E4M3 codes)
  constexpr int KW = FP8 ? D / 64 : KC;
  static_assert(FP8 || 2 * KW == NV, "bf16 K rows use the V copy's instruction count");
  constexpr int kInFlight = 2;
  struct Chunk {
    u32x4 k[2][KW];
    u32x4 v[NV];
  };
  // Element offset of the first row of the 16-key group starting at key g0 (clamped to the
  // last visible group). A 16-key group lies in one block (block_size is a multiple of 16);
  // the block index comes from the host's 32.32 reciprocal of block_size / 16.
  const int last_group = last_key & ~15;
  const uint32_t block_elems = (uint32_t)(p.block_size * p.num_kv_heads * D);   // < 2^31
  const int kv_row = p.num_kv_heads * D;
  auto group_off = [&](int g0, int* first_key) __attribute__((always_inline)) {
    g0 = min(g0, last_group);
    *first_key = g0;
    const uint32_t bidx = (uint32_t)(((uint64_t)(uint32_t)(g0 >> 4) * p.group_recip) >> 32);
    const int32_t blk = block_of(bidx);
    return (uint64_t)(uint32_t)blk * block_elems +
           (uint32_t)((g0 - (int)bidx * p.block_size) * kv_row + kvh * D);
  };
  // keys past the wave's range load a valid row (clamped); their scores are masked, so they
  // add 0 * (finite V) and need no zeroing
  auto load_chunk = [&](Chunk& ch, int kb) __attribute__((always_inline)) {
    if constexpr (FP8) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        int g0;
        const uint64_t base = group_off(kb + 16 * t2, &g0);
        const kv_t* src = kcache + base + (uint32_t)(min(li, last_key - g0) * kv_row + 16 * G);
#pragma unroll
        for (int c = 0; c < KW; ++c) ch.k[t2][c] = *reinterpret_cast<const u32x4*>(src + 64 * c);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int row = j * RPI + v_row;               // as for V below
        int g0;
        const uint64_t base = group_off(kb + (j * RPI / 16) * 16, &g0);
        ch.k[j / KW][j % KW] = *reinterpret_cast<const u32x4*>(
            kcache + base + (uint32_t)(min(row % 16, last_key - g0) * kv_row + EPL * v_chunk));
      }
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int row = j * RPI + v_row;                 // row in the chunk; its 16-key group
      int g0;                                          // is uniform across the instruction
      const uint64_t base = group_off(kb + (j * RPI / 16) * 16, &g0);
      ch.v[j] = *reinterpret_cast<const u32x4*>(
          vcache + base + (uint32_t)(min(row % 16, last_key - g0) * kv_row + EPL * v_chunk));
    }
  };

  const float c_log2 = p.scale * kLog2e;
  m_run = -INFINITY;
  l_run = 0.f;
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) o[dc] = floatx4{0.f, 0.f, 0.f, 0.f};

  // consume chunk ci held in ch; after its QK^T MFMAs, refill ch with chunk ci + 2
  // Refill (a std::integral_constant<bool, ...>): whether ch is refilled; kept a compile-time
  // choice so that every load in the main loop is unconditional and the compiler's wait
  // counts see a fixed number of loads in flight (a refill under a run-time condition made
  // it wait for both buffers before each chunk, leaving one chunk in flight instead of two)
  auto consume = [&](Chunk& ch, int ci, auto refill) __attribute__((always_inline)) {
    const int kb = c_base + (c_first + ci) * kChunk;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      __bf16* dst = &sVw[(j * RPI + v_row) * RS + EPL * v_chunk];
      if constexpr (FP8) {
        *reinterpret_cast<bf16x8*>(dst) = fp8x8_to_bf16x8(ch.v[j][0], ch.v[j][1]);
        *reinterpret_cast<bf16x8*>(dst + 8) = fp8x8_to_bf16x8(ch.v[j][2], ch.v[j][3]);
      } else {
        *reinterpret_cast<bf16x8*>(dst) = __builtin_bit_cast(bf16x8, ch.v[j]);
      }
    }
    if constexpr (!FP8) {
      // K rows into the K tile; once both tiles are written the chunk's registers are free,
      // so the chunk after next is requested before the MFMAs
#pragma unroll
      for (int j = 0; j < NV; ++j)
        *reinterpret_cast<bf16x8*>(&sKw[(j * RPI + v_row) * KRS + EPL * v_chunk]) =
            __builtin_bit_cast(bf16x8, ch.k[j / KW][j % KW]);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the writes land before any read
      if constexpr (decltype(refill)::value) load_chunk(ch, kb + kInFlight * kChunk);
    }
    floatx4 sc[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        bf16x8 ka;
        if constexpr (FP8)
          ka = fp8x8_to_bf16x8(ch.k[t2][c / 2][2 * (c % 2)], ch.k[t2][c / 2][2 * (c % 2) + 1]);
        else   // the A operand: lane (G, li) holds key 16 t2 + li, d = 32c + 8G .. +7
          ka = *reinterpret_cast<const bf16x8*>(&sKw[(16 * t2 + li) * KRS + 32 * c + 8 * G]);
        acc = mfma16x16x32(ka, qf[c], acc);
      }
      sc[t2] = acc;
    }
    if constexpr (FP8) {
      if constexpr (decltype(refill)::value) load_chunk(ch, kb + kInFlight * kChunk);
    }
    if (kb < w_begin || kb + kChunk > w_end) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = kb + 16 * t2 + 4 * G + e;
          if (j < w_begin || j >= w_end) sc[t2][e] = -INFINITY;
        }
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = column_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2((m_run - m_use) * c_log2);
    const float mc = m_use * c_log2;
    float lsum = 0.f;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pv = fast_exp2(fmaf(sc[t2][e], c_log2, -mc));
        sc[t2][e] = pv;
        lsum += pv;
      }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
    const bf16x8 pb = pack_bf16x8(sc[0], sc[1]);

    // the LDS writes above must land before other lanes of this wave read them
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int r0 = 4 * G + li / 4;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const int col = 16 * dc + 4 * (li % 4);
      const bf16x8 va = concat(lds_read_tr16(&sVw[r0 * RS + col]),
                               lds_read_tr16(&sVw[(r0 + 16) * RS + col]));
      o[dc] = mfma16x16x32(va, pb, o[dc] * alpha);
    }
    // the next chunk's LDS writes must not pass these reads
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };

  // kInFlight = 2 chunks in flight per wave (4 for E4M3 measured no faster than 2). The chunk
  // count is rounded up to even: the extra chunk lies past w_end (clamped loads, masked
  // scores), so every pair of chunks is one pass of the loop with both refills issued; the
  // last pair refills nothing.
  static_assert(kInFlight == 2, "the loop below consumes chunks in pairs");
  if (n_chunks == 0) return;
  const int n_pairs = (n_chunks + 1) / 2;
  const int k0 = c_base + c_first * kChunk;
  auto after_real = [&](int ci) __attribute__((always_inline)) {
    if (ci < n_chunks) after(k0 + ci * kChunk);
  };
  Chunk buf[kInFlight];
  load_chunk(buf[0], k0);
  load_chunk(buf[1], k0 + kChunk);
  for (int pr = 0; pr + 1 < n_pairs; ++pr) {
    consume(buf[0], 2 * pr, std::true_type{});
    after_real(2 * pr);
    consume(buf[1], 2 * pr + 1, std::true_type{});
    after_real(2 * pr + 1);
  }
  consume(buf[0], 2 * n_pairs - 2, std::false_type{});
  after_real(2 * n_pairs - 2);
  consume(buf[1], 2 * n_pairs - 1, std::false_type{});
  after_real(2 * n_pairs - 1);
}

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
