// Prefill attention kernel, bf16 in / fp32 accumulate, for gfx950.
//
// Method (vLLM FlashAttention page, sections "들어가며" and "논문 핵심 내용"): Q, K and V are
// brought on chip tile by tile, the softmax is carried online with a running max and a running
// sum, and only the final rows (plus their log-sum-exp) are written, so no score matrix ever
// reaches HBM. K/V rows are read through the block table from the paged cache of the
// FlashAttentionBackend section; GQA follows num_queries_per_kv of the FlashAttentionImpl
// section; causal and sliding-window masks follow the RBLN "Attention 모드" page.
//
// Work split: one workgroup = 8 waves of one (request, q head); each wave owns 32 query rows,
// one 32-wide MFMA column block, so a workgroup covers 256 rows and every K/V tile brought on
// chip serves 256 queries. KV is walked in 64-key tiles through two LDS buffers:
//   * all 512 threads gather the next tile's K and V rows (16-byte loads; the block of each
//     16-key group is a wave-uniform scalar lookup) into registers while the current tile is
//     consumed, then store them into the other buffer; one barrier per tile;
//   * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 (K from LDS as the A operand, Q^T held in
//     registers as the B operand). On gfx950 this shape sustains about 1.6x the bf16 rate of
//     the 16x16x32 shape. Each lane holds 16 keys of one query, so the row max and row sum
//     need one v_permlane32_swap;
//   * P^T stays in registers and is already in the B-operand layout of the PV MFMA;
//   * O^T += V^T . P^T, with V^T read straight from the row-major V tile by
//     ds_read_b64_tr_b16, so no transpose pass is needed;
//   * each lane owns one query column of O^T, so the softmax rescale is lane-local. The
//     reference max is only moved when a new score exceeds it by more than 2^8 (in exp2
//     units): the result O / l is the same for any reference, the skipped rescales save most
//     of the per-tile VALU work, and p = 2^(s*c - m*c) stays <= 256.
//
// v_mfma_f32_32x32x16_bf16 lane layout (lane l, h = l / 32), checked on gfx950:
//   A (32 x 16): element e of lane l is A[l % 32][8h + e]
//   B (16 x 32): element e of lane l is B[8h + e][l % 32]
//   C (32 x 32): element e of lane l is C[8(e / 4) + 4h + e % 4][l % 32]
#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kRows = 32;     // query rows per wave
constexpr float kRescaleLog2 = 8.f;
constexpr int kWaves = 8;                    // waves per workgroup (2 per SIMD)
constexpr int kBC = 64;                      // keys per KV tile
constexpr int kThreads = kWaves * kWave;
constexpr int kBR = kWaves * kRows;          // query rows per workgroup
constexpr int kKT = kBC / 32;                // 32-key MFMA tiles per KV tile

typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ floatx16 mfma32x32x16(const bf16x8& a, const bf16x8& b,
                                                 const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D, bool CAUSAL, bool WINDOW>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(const PrefillParams p) {
  constexpr int RS = D + 16;          // LDS row stride in bf16 (padding against bank conflicts)
  constexpr int KC = D / 16;          // 16-deep k-chunks of the QK^T contraction
  constexpr int DC = D / 32;          // 32-wide d chunks of O^T
  constexpr int TPR = D / 8;          // threads per K/V row in the gather (16 bytes each)
  constexpr int RPP = kThreads / TPR;  // rows per gather pass
  constexpr int NP = kBC / RPP;       // gather passes per tile
  constexpr int RPW = kWave / TPR;    // rows per wave per pass (4 or 8: divides 16)
  constexpr int TILE = kBC * RS;

  __shared__ __attribute__((aligned(16))) __bf16 sK[2 * TILE];
  __shared__ __attribute__((aligned(16))) __bf16 sV[2 * TILE];

  const int r = p.seq_begin + blockIdx.z;
  const int hq = blockIdx.y;
  const int qt = gridDim.x - 1 - blockIdx.x;   // longest (causal) tiles are dispatched first
  const int q_start = p.qsl[r];
  const int ql = p.qsl[r + 1] - q_start;
  if (qt * kBR >= ql) return;
  const int sl = p.seq_lens[r];
  const int cl = sl - ql;
  const int kvh = hq / (p.num_heads / p.num_kv_heads);

  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int lane = tid % kWave;
  const int h = lane / 32;            // half-wave
  const int lq = lane % 32;           // query column of this lane

  const __bf16* __restrict__ q = static_cast<const __bf16*>(p.q);
  const __bf16* __restrict__ kcache = static_cast<const __bf16*>(p.kv);
  const __bf16* __restrict__ vcache = kcache + p.v_offset;
  const int32_t* __restrict__ bt = p.block_table + (int64_t)r * p.max_blocks;
  const int64_t row_stride = (int64_t)p.num_heads * D;   // q/out stride between tokens

  // ---- Q^T (B operand): lane l holds query lq, d = 16c + 8h .. +7
  const int wrow0 = qt * kBR + w * kRows;                // first query row of this wave
  bf16x8 qf[KC];
  {
    const int row = min(wrow0 + lq, ql - 1);             // rows past ql: any valid row
    const __bf16* src = q + (int64_t)(q_start + row) * row_stride + (int64_t)hq * D + 8 * h;
#pragma unroll
    for (int c = 0; c < KC; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(src + 16 * c);
  }

  // ---- KV range of the workgroup and of this wave
  const int row_lo = qt * kBR;
  const int row_hi = min(ql, row_lo + kBR) - 1;
  const int kv_hi = CAUSAL ? min(sl, cl + row_hi + 1) : sl;
  const int kv_lo = WINDOW ? max(0, cl + row_lo - p.window + 1) : 0;
  const int t_begin = kv_lo / kBC;
  const int t_end = (kv_hi + kBC - 1) / kBC;
  const int w_row_lo = wrow0;
  const int w_row_hi = min(ql, wrow0 + kRows) - 1;
  const bool wave_active = w_row_lo <= w_row_hi;
  const int w_kv_hi = CAUSAL ? min(sl, cl + w_row_hi + 1) : sl;
  const int w_kv_lo = WINDOW ? max(0, cl + w_row_lo - p.window + 1) : 0;

  // ---- gather: thread -> (row in pass, 16-byte chunk). The rows one wave gathers in a pass
  // lie in one 16-key group, and a 16-key group lies in one cache block (block_size is a
  // multiple of 16), so the block lookup is wave-uniform: scalar loads of the block table,
  // one tile ahead of the K/V rows. Block index of group g: g / (block_size / 16), from the
  // host's 32.32 reciprocal.
  const int g_row = tid / TPR;
  const int g_chunk = tid % TPR;
  const uint32_t block_elems = (uint32_t)(p.block_size * p.num_kv_heads * D);   // < 2^31
  const int kv_row = p.num_kv_heads * D;
  const int groups_per_block = p.block_size / 16;
  const int last_group = (sl - 1) >> 4;
  uint64_t blk_off[NP];     // element offset of the 16-key group each pass reads (uniform)
  auto fetch_blocks = [&](int tile) {
    int grp[NP];
    uint32_t bidx[NP];
    int32_t blk[NP];
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {   // all table loads first, then one wait
      grp[pp] = min(__builtin_amdgcn_readfirstlane((tile * kBC + pp * RPP + w * RPW) >> 4),
                    last_group);                     // groups past seq_len: any valid group
      bidx[pp] = (uint32_t)(((uint64_t)(uint32_t)grp[pp] * p.group_recip) >> 32);
      blk[pp] = bt[bidx[pp]];
    }
#pragma unroll
    for (int pp = 0; pp < NP; ++pp)
      blk_off[pp] = (uint64_t)(uint32_t)blk[pp] * block_elems +
                    (uint32_t)((grp[pp] - (int)bidx[pp] * groups_per_block) * 16 * kv_row);
  };
  u32x4 kreg[NP], vreg[NP];
  auto gather = [&]() {       // K/V rows of the tile whose groups are in blk_off
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const uint32_t lane_off =
          (uint32_t)((((pp * RPP + w * RPW) & 15) + lane / TPR) * kv_row + kvh * D + g_chunk * 8);
      kreg[pp] = *reinterpret_cast<const u32x4*>(kcache + blk_off[pp] + lane_off);
      vreg[pp] = *reinterpret_cast<const u32x4*>(vcache + blk_off[pp] + lane_off);
    }
  };
  auto stash = [&](int buf, int tile) {
    if (tile * kBC + kBC > sl) {                     // tail tile: zero keys past seq_len
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        if (tile * kBC + pp * RPP + g_row >= sl) {
          kreg[pp] = u32x4{0, 0, 0, 0};
          vreg[pp] = u32x4{0, 0, 0, 0};
        }
      }
    }
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      *reinterpret_cast<u32x4*>(&sK[buf * TILE + (pp * RPP + g_row) * RS + g_chunk * 8]) = kreg[pp];
      *reinterpret_cast<u32x4*>(&sV[buf * TILE + (pp * RPP + g_row) * RS + g_chunk * 8]) = vreg[pp];
    }
  };

  const float c_log2 = p.scale * kLog2e;
  float m_ref = -INFINITY;
  float l_run = 0.f;        // per-lane partial row sum (fp32: the lse needs it unrounded)
  floatx16 o[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dc][e] = 0.f;

  if (t_begin < t_end) {
    fetch_blocks(t_begin);
    gather();
    if (t_begin + 1 < t_end) fetch_blocks(t_begin + 1);
    stash(0, t_begin);
  }
  __syncthreads();
  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    const bool more = t + 1 < t_end;
    if (more) {                  // in flight while this tile is consumed
      gather();
      if (t + 2 < t_end) fetch_blocks(t + 2);
    }

    const int kb = t * kBC;
    if (wave_active && kb < w_kv_hi && kb + kBC > w_kv_lo) {
      const __bf16* tK = sK + buf * TILE;
      const __bf16* tV = sV + buf * TILE;
      // S^T: sc[kt] element e holds key kb + 32kt + 8(e/4) + 4h + e%4 of query column lq
      floatx16 sc[kKT];
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt) {
        const __bf16* krow = &tK[(kt * 32 + lq) * RS + 8 * h];
        floatx16 acc;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
        for (int c = 0; c < KC; ++c)
          acc = mfma32x32x16(*reinterpret_cast<const bf16x8*>(krow + 16 * c), qf[c], acc);
        sc[kt] = acc;
      }

      const bool need_mask = (kb + kBC > sl) || (CAUSAL && kb + kBC - 1 > cl + w_row_lo) ||
                             (WINDOW && kb < cl + w_row_hi - p.window + 1);
      if (need_mask) {
        const int pos = cl + wrow0 + lq;             // absolute position of this query
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int j = kb + 32 * kt + 8 * (e / 4) + 4 * h + (e % 4);
            bool vis = j < sl;
            if (CAUSAL) vis = vis && (j <= pos);
            if (WINDOW) vis = vis && (j >= pos - p.window + 1);
            if (!vis) sc[kt][e] = -INFINITY;
          }
      }

      // online softmax with a lazily moved reference max, one query column per lane pair
      float mx = __builtin_fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
      for (int x = 2; x < 16 * kKT; x += 2)
        mx = __builtin_fmaxf(__builtin_fmaxf(mx, sc[x / 16][x % 16]), sc[x / 16][x % 16 + 1]);
      mx = max_xor32(mx);
      // move the reference when the tile max exceeds it by more than 2^kRescaleLog2
      // (always on a column's first visible key, where m_ref is -inf)
      const bool move = (mx - m_ref) * c_log2 > kRescaleLog2;
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
        // alpha is 0 when m_ref was -inf; columns that keep their reference use 1
        const float alpha = move ? fast_exp2((m_ref - mx) * c_log2) : 1.f;
        if (move) m_ref = mx;
        l_run *= alpha;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) o[dc] *= alpha;
      }
      const float mc = (m_ref == -INFINITY) ? 0.f : m_ref * c_log2;
      float lsum = 0.f;
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          sc[kt][e] = fast_exp2(fmaf(sc[kt][e], c_log2, -mc));
          lsum += sc[kt][e];
        }
      l_run += lsum;

      // O^T += V^T . P^T, one MFMA per 16 keys: MFMA (kt, g) contracts keys
      // kb + 32kt + 16g + 8(j/4) + 4h + j%4 at k = 8h + j. P^T is elements 8g .. 8g+7 of
      // sc[kt]; V^T comes from two transposing reads of 4 rows each.
      const int col0 = 16 * ((lane / 16) % 2) + 4 * (lane % 4);
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const floatx4 lo = {sc[kt][8 * g + 0], sc[kt][8 * g + 1], sc[kt][8 * g + 2],
                              sc[kt][8 * g + 3]};
          const floatx4 hi = {sc[kt][8 * g + 4], sc[kt][8 * g + 5], sc[kt][8 * g + 6],
                              sc[kt][8 * g + 7]};
          const bf16x8 pb = pack_bf16x8(lo, hi);
          const int r0 = 32 * kt + 16 * g + 4 * h + (lane % 16) / 4;
#pragma unroll
          for (int dc = 0; dc < DC; ++dc) {
            const int col = 32 * dc + col0;
            const bf16x8 va = concat(lds_read_tr16(&tV[r0 * RS + col]),
                                     lds_read_tr16(&tV[(r0 + 8) * RS + col]));
            o[dc] = mfma32x32x16(va, pb, o[dc]);
          }
        }
    }
    if (more) stash(buf ^ 1, t + 1);
    __syncthreads();
  }

  // ---- epilogue: O / l and lse = scale * m + ln l
  const float l_tot = add_xor32(l_run);
  const int row = wrow0 + lq;
  if (row < ql) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __bf16* dst = static_cast<__bf16*>(p.out) + (int64_t)(q_start + row) * row_stride +
                  (int64_t)hq * D + 4 * h;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        bf16x4 v;
        v[0] = to_bf16(o[dc][4 * e4 + 0] * inv);
        v[1] = to_bf16(o[dc][4 * e4 + 1] * inv);
        v[2] = to_bf16(o[dc][4 * e4 + 2] * inv);
        v[3] = to_bf16(o[dc][4 * e4 + 3] * inv);
        *reinterpret_cast<bf16x4*>(dst + 32 * dc + 8 * e4) = v;
      }
    if (p.lse != nullptr && h == 0) {
      p.lse[(int64_t)(q_start + row) * p.num_heads + hq] =
          l_tot > 0.f ? p.scale * m_ref + __logf(l_tot) : -INFINITY;
    }
  }
}

template <int D, bool CAUSAL, bool WINDOW>
hipError_t launch(const PrefillParams& p, hipStream_t stream) {
  const dim3 grid((p.max_query_len + kBR - 1) / kBR, p.num_heads, p.num_seqs);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, WINDOW>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mask(const PrefillParams& p, hipStream_t stream) {
  if (p.window > 0) return launch<D, true, true>(p, stream);
  if (p.causal) return launch<D, true, false>(p, stream);
  return launch<D, false, false>(p, stream);
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream) {
  if (p.num_seqs <= 0 || p.max_query_len <= 0) return hipSuccess;
  return p.head_size == 64 ? launch_mask<64>(p, stream) : launch_mask<128>(p, stream);
}

}  // namespace attn
