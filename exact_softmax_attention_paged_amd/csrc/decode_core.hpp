// Per-wave pieces of the split-KV decode, shared by the decode kernels and the mixed
// prefill + decode kernel (gfx950): the Q^T fragment, one wave's online-softmax stream over a
// run of a request's keys, and a whole decode request streamed by one wave.
#pragma once
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace dec {

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
// the request's b-th block of this pass. Updates, per lane (G, li), the running max m_run and
// this lane's share of the running sum l_run (scores of column li; m_run is the same in
// every lane of a column), and O^T: o[dc][e] = sum_j p_j V[j][16 dc + 4 G + e] for q head
// li, unnormalised (init_state starts them empty). after(kb) runs after the chunk at key kb.
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
  // add 0 * (finite V) and need no zeroing. Every K/V load is non-temporal (nt): each row is
  // read once per kv head, and streaming hints keep it from displacing cached lines - on
  // gfx950 the decode stream runs 6-10 % faster with them (5.80 -> 6.39 TB/s on the paged GQA
  // decode) and it leaves the L2 to the prefill rows it runs beside.
  auto load_chunk = [&](Chunk& ch, int kb) __attribute__((always_inline)) {
    if constexpr (FP8) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        int g0;
        const uint64_t base = group_off(kb + 16 * t2, &g0);
        const kv_t* src = kcache + base + (uint32_t)(min(li, last_key - g0) * kv_row + 16 * G);
#pragma unroll
        for (int c = 0; c < KW; ++c)
          ch.k[t2][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + 64 * c));
      }
    } else {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int row = j * RPI + v_row;               // as for V below
        int g0;
        const uint64_t base = group_off(kb + (j * RPI / 16) * 16, &g0);
        ch.k[j / KW][j % KW] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
            kcache + base + (uint32_t)(min(row % 16, last_key - g0) * kv_row + EPL * v_chunk)));
      }
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int row = j * RPI + v_row;                 // row in the chunk; its 16-key group
      int g0;                                          // is uniform across the instruction
      const uint64_t base = group_off(kb + (j * RPI / 16) * 16, &g0);
      ch.v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          vcache + base + (uint32_t)(min(row % 16, last_key - g0) * kv_row + EPL * v_chunk)));
    }
  };

  const float c_log2 = p.scale * kLog2e;

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

__device__ __forceinline__ void init_state(float& m_run, float& l_run, floatx4* o, int dcs) {
  m_run = -INFINITY;
  l_run = 0.f;
  for (int dc = 0; dc < dcs; ++dc) o[dc] = floatx4{0.f, 0.f, 0.f, 0.f};
}

// The cache blocks of a run of at most 64 blocks of request r (pass blocks b_first ..), one
// per lane, read back with v_readlane at a wave-uniform index.
struct LaneBlocks {
  int32_t blk;
  int b_first;
  __device__ __forceinline__ int32_t operator()(uint32_t bidx) const {
    return __builtin_amdgcn_readlane(blk, (int)(bidx - b_first));
  }
};
__device__ __forceinline__ LaneBlocks lane_blocks(const DecodeParams& p, int r, int b_first,
                                                  int n_blk) {
  const int lane = threadIdx.x % kWave;
  const int32_t* __restrict__ bt = p.block_table + (int64_t)r * p.max_blocks + p.kv_skip_blocks;
  return LaneBlocks{lane < n_blk ? bt[b_first + lane] : 0, b_first};
}

// One wave streams every visible key of decode request r for the q heads of (kv head, head
// group) hw, 64 cache blocks at a time (their ids one per lane), and writes the request's
// output and lse directly: no partitions and no merge. sVw / sKw: the wave's LDS tiles.
template <int D>
__device__ __forceinline__ void decode_request_wave(const DecodeParams& p, int r, int hw,
                                                    __bf16* sVw, __bf16* sKw) {
  const int lane = threadIdx.x % kWave;
  const int G = lane / 16;
  const int li = lane % 16;
  const int group = p.num_heads / p.num_kv_heads;
  const int head_groups = (group + 15) / 16;
  const int kvh = hw / head_groups;
  const int hg = hw % head_groups;
  const int nh = min(16, group - hg * 16);
  const int h0 = kvh * group + hg * 16;
  const int tok = p.qsl[r];
  const int sl = p.seq_lens[r] - p.kv_skip_blocks * p.block_size;
  const int lo = p.window > 0 ? max(0, sl - p.window) : 0;
  bf16x8 qf[D / 32];
  load_q_frag<D, false>(p, tok, h0, nh, qf);
  float m_run, l_run;
  floatx4 o[D / 16];
  init_state(m_run, l_run, o, D / 16);
  const int seg_keys = 64 * p.block_size;
  for (int s0 = lo / seg_keys * seg_keys; s0 < sl; s0 += seg_keys) {
    const int k_end = min(sl, s0 + seg_keys);
    const int b_first = s0 / p.block_size;
    const LaneBlocks lb = lane_blocks(p, r, b_first, (k_end - 1) / p.block_size - b_first + 1);
    stream_keys<D, false>(p, kvh, qf, s0, max(lo, s0), k_end, k_end - 1, lb, sVw, sKw, m_run,
                          l_run, o, [](int) {});
  }
  const float l = column_sum(l_run);
  if (li >= nh) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t row = (int64_t)tok * p.num_heads + h0 + li;
  __bf16* dst = static_cast<__bf16*>(p.out) + row * D;
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) {
    const floatx4 v = o[dc] * inv;
    bf16x4 b4;
#pragma unroll
    for (int e = 0; e < 4; ++e) b4[e] = to_bf16(v[e]);
    *reinterpret_cast<bf16x4*>(dst + 16 * dc + 4 * G) = b4;
  }
  if (p.lse != nullptr && G == 0) p.lse[row] = l > 0.f ? p.scale * m_run + __logf(l) : -INFINITY;
}

}  // namespace dec
}  // namespace attn
