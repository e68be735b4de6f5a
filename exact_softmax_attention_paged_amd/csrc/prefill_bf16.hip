// Prefill attention kernel, bf16 in / fp32 accumulate, for gfx950.
//
// Method (vLLM FlashAttention page, sections "들어가며" and "논문 핵심 내용"): Q, K and V are
// brought on chip tile by tile, the softmax is carried online with a running max and a running
// sum, and only the final rows (plus their log-sum-exp) are written, so no score matrix ever
// reaches HBM. K/V rows are read through the block table from the paged cache of the
// FlashAttentionBackend section; GQA follows num_queries_per_kv of the FlashAttentionImpl
// section; causal and sliding-window masks follow the RBLN "Attention 모드" page.
//
// Work split: one workgroup = 4 waves of one (request, q head); each wave owns ROWS = 16*QS
// query rows (QS 16-row MFMA columns), so a workgroup covers 4*ROWS rows. KV is walked in
// 64-key tiles through two LDS buffers:
//   * all 256 threads gather the next tile's K and V rows (16-byte loads, block index from a
//     host-computed reciprocal) into registers while the current tile is consumed, then store
//     them into the other buffer; one barrier per tile;
//   * S^T = K . Q^T on v_mfma_f32_16x16x32_bf16 (K from LDS as the A operand, Q^T held in
//     registers as the B operand), so each lane holds 4 keys of one query: the row max and row
//     sum need only the 4 lanes of a column (v_permlane16/32_swap);
//   * P^T stays in registers and is already in the B-operand layout of the next MFMA;
//   * O^T += V^T . P^T, with V^T read straight from the row-major V tile by
//     ds_read_b64_tr_b16, so no transpose pass is needed;
//   * each lane owns one query column of O^T, so the softmax rescale is lane-local. The
//     reference max is only moved when a new score exceeds it by more than 2^8 (in exp2
//     units): the result O / l is the same for any reference, the skipped rescales save most
//     of the per-tile VALU work, and p = 2^(s*c - m*c) stays <= 256.
#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kBC = 64;       // keys per KV tile
constexpr int kWaves = 4;
constexpr float kRescaleLog2 = 8.f;


template <int D, int QS, bool CAUSAL, bool WINDOW>
__global__ __launch_bounds__(256, QS == 4 ? 1 : 2) void prefill_bf16_kernel(const PrefillParams p) {
  constexpr int ROWS = 16 * QS;       // query rows per wave
  constexpr int BR = kWaves * ROWS;   // query rows per workgroup
  constexpr int RS = D + 16;          // LDS row stride in bf16 (padding against bank conflicts)
  constexpr int KC = D / 32;          // k-chunks of the QK^T contraction
  constexpr int DC = D / 16;          // 16-wide d chunks of O^T
  constexpr int TPR = D / 8;          // threads per K/V row in the gather (16 bytes each)
  constexpr int RPP = 256 / TPR;      // rows per gather pass
  constexpr int NP = kBC / RPP;       // gather passes per tile
  constexpr int TILE = kBC * RS;

  __shared__ __attribute__((aligned(16))) __bf16 sK[2 * TILE];
  __shared__ __attribute__((aligned(16))) __bf16 sV[2 * TILE];

  const int r = p.seq_begin + blockIdx.z;
  const int h = blockIdx.y;
  const int qt = gridDim.x - 1 - blockIdx.x;   // longest (causal) tiles are dispatched first
  const int q_start = p.qsl[r];
  const int ql = p.qsl[r + 1] - q_start;
  if (qt * BR >= ql) return;
  const int sl = p.seq_lens[r];
  const int cl = sl - ql;
  const int kvh = h / (p.num_heads / p.num_kv_heads);

  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int lane = tid % kWave;
  const int G = lane / 16;
  const int li = lane % 16;

  const __bf16* __restrict__ q = static_cast<const __bf16*>(p.q);
  const __bf16* __restrict__ kcache = static_cast<const __bf16*>(p.kv);
  const __bf16* __restrict__ vcache = kcache + p.v_offset;
  const int32_t* __restrict__ bt = p.block_table + (int64_t)r * p.max_blocks;
  const int64_t row_stride = (int64_t)p.num_heads * D;   // q/out stride between tokens

  // ---- Q^T fragments (B operand): lane (G, li) holds query li, d = 32c + 8G .. +7
  bf16x8 qf[QS][KC];
  const int wrow0 = qt * BR + w * ROWS;                 // first query row of this wave
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    const int row = min(wrow0 + s * 16 + li, ql - 1);   // rows past ql: any valid row
#pragma unroll
    for (int c = 0; c < KC; ++c)
      qf[s][c] = *reinterpret_cast<const bf16x8*>(q + (int64_t)(q_start + row) * row_stride +
                                                  (int64_t)h * D + 32 * c + 8 * G);
  }

  // ---- KV range of the workgroup and of this wave
  const int row_lo = qt * BR;
  const int row_hi = min(ql, row_lo + BR) - 1;
  const int kv_hi = CAUSAL ? min(sl, cl + row_hi + 1) : sl;
  const int kv_lo = WINDOW ? max(0, cl + row_lo - p.window + 1) : 0;
  const int t_begin = kv_lo / kBC;
  const int t_end = (kv_hi + kBC - 1) / kBC;
  const int w_row_lo = wrow0;
  const int w_row_hi = min(ql, wrow0 + ROWS) - 1;
  const bool wave_active = w_row_lo <= w_row_hi;
  const int w_kv_hi = CAUSAL ? min(sl, cl + w_row_hi + 1) : sl;
  const int w_kv_lo = WINDOW ? max(0, cl + w_row_lo - p.window + 1) : 0;

  // ---- gather: thread -> (row in pass, 16-byte chunk). The rows one wave gathers in a pass
  // lie in one 16-key group, and a 16-key group lies in one cache block (block_size is a
  // multiple of 16), so the block lookup is wave-uniform: scalar loads of the block table,
  // one tile ahead of the K/V rows. Block index of group g: g / (block_size / 16), computed
  // with the host's 32.32 reciprocal.
  constexpr int RPW = kWave / TPR;    // rows per wave per pass (4 or 8: divides 16)
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
  float m_ref[QS];
  floatx4 o[QS][DC];
  float l_run[QS];     // per-lane partial row sums (fp32: the lse needs them unrounded)
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    m_ref[s] = -INFINITY;
    l_run[s] = 0.f;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) o[s][dc] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

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
      // S^T tiles: sc[s][kt] holds keys kb + 16kt + 4G + e of query column li
      floatx4 sc[QS][4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        bf16x8 kf[KC];
#pragma unroll
        for (int c = 0; c < KC; ++c)
          kf[c] = *reinterpret_cast<const bf16x8*>(&tK[(kt * 16 + li) * RS + 32 * c + 8 * G]);
#pragma unroll
        for (int s = 0; s < QS; ++s) {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < KC; ++c) acc = mfma16x16x32(kf[c], qf[s][c], acc);
          sc[s][kt] = acc;
        }
      }

      const bool need_mask = (kb + kBC > sl) || (CAUSAL && kb + kBC - 1 > cl + w_row_lo) ||
                             (WINDOW && kb < cl + w_row_hi - p.window + 1);
      if (need_mask) {
#pragma unroll
        for (int s = 0; s < QS; ++s) {
          const int pos = cl + wrow0 + s * 16 + li;   // absolute position of this query
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int j = kb + kt * 16 + 4 * G + e;
              bool vis = j < sl;
              if (CAUSAL) vis = vis && (j <= pos);
              if (WINDOW) vis = vis && (j >= pos - p.window + 1);
              if (!vis) sc[s][kt][e] = -INFINITY;
            }
        }
      }

      // online softmax with a lazily moved reference max, one query column per lane
#pragma unroll
      for (int s = 0; s < QS; ++s) {
        float mx = __builtin_fmaxf(sc[s][0][0], sc[s][0][1]);
#pragma unroll
        for (int x = 2; x < 16; x += 2)
          mx = __builtin_fmaxf(__builtin_fmaxf(mx, sc[s][x / 4][x % 4]), sc[s][x / 4][x % 4 + 1]);
        mx = column_max(mx);
        // move the reference when the tile max exceeds it by more than 2^kRescaleLog2
        // (always on the first visible tile, where m_ref is -inf)
        const bool move = (mx - m_ref[s]) * c_log2 > kRescaleLog2;
        if (__builtin_amdgcn_ballot_w64(move) != 0) {
          // alpha is 0 when m_ref was -inf; columns that keep their reference use 1
          const float alpha = move ? fast_exp2((m_ref[s] - mx) * c_log2) : 1.f;
          if (move) m_ref[s] = mx;
          l_run[s] *= alpha;
#pragma unroll
          for (int dc = 0; dc < DC; ++dc) o[s][dc] *= alpha;
        }
        const float mc = (m_ref[s] == -INFINITY) ? 0.f : m_ref[s] * c_log2;
        float lsum = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sc[s][kt][e] = fast_exp2(fmaf(sc[s][kt][e], c_log2, -mc));
            lsum += sc[s][kt][e];
          }
        l_run[s] += lsum;
      }

      // O^T += V^T . P^T over two 32-key halves
#pragma unroll
      for (int hk = 0; hk < 2; ++hk) {
        bf16x8 pb[QS];
#pragma unroll
        for (int s = 0; s < QS; ++s) pb[s] = pack_bf16x8(sc[s][2 * hk], sc[s][2 * hk + 1]);
        const int r0 = 32 * hk + 4 * G + li / 4;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          const int col = 16 * dc + 4 * (li % 4);
          const bf16x8 va = concat(lds_read_tr16(&tV[r0 * RS + col]),
                                   lds_read_tr16(&tV[(r0 + 16) * RS + col]));
#pragma unroll
          for (int s = 0; s < QS; ++s) o[s][dc] = mfma16x16x32(va, pb[s], o[s][dc]);
        }
      }
    }
    if (more) stash(buf ^ 1, t + 1);
    __syncthreads();
  }

  // ---- epilogue: O / l and lse = scale * m + ln l
  __bf16* __restrict__ out = static_cast<__bf16*>(p.out);
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    const float l_tot = column_sum(l_run[s]);
    const int row = wrow0 + s * 16 + li;
    if (row >= ql) continue;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __bf16* dst = out + (int64_t)(q_start + row) * row_stride + (int64_t)h * D + 4 * G;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      bf16x4 v;
      v[0] = to_bf16(o[s][dc][0] * inv);
      v[1] = to_bf16(o[s][dc][1] * inv);
      v[2] = to_bf16(o[s][dc][2] * inv);
      v[3] = to_bf16(o[s][dc][3] * inv);
      *reinterpret_cast<bf16x4*>(dst + 16 * dc) = v;
    }
    if (p.lse != nullptr && G == 0) {
      p.lse[(int64_t)(q_start + row) * p.num_heads + h] =
          l_tot > 0.f ? p.scale * m_ref[s] + __logf(l_tot) : -INFINITY;
    }
  }
}

template <int D, int QS, bool CAUSAL, bool WINDOW>
hipError_t launch(const PrefillParams& p, hipStream_t stream) {
  constexpr int BR = kWaves * 16 * QS;
  const dim3 grid((p.max_query_len + BR - 1) / BR, p.num_heads, p.num_seqs);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, QS, CAUSAL, WINDOW>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D, int QS>
hipError_t launch_mask(const PrefillParams& p, hipStream_t stream) {
  if (p.window > 0) return launch<D, QS, true, true>(p, stream);
  if (p.causal) return launch<D, QS, true, false>(p, stream);
  return launch<D, QS, false, false>(p, stream);
}

template <int D>
hipError_t launch_rows(const PrefillParams& p, hipStream_t stream) {
  // 32 rows per wave. 64 rows per wave (QS = 4, one wave per SIMD) halves the LDS bytes per
  // MFMA but measured 27 % (d 128) to 48 % (d 64) slower on the workloads here: with a single
  // wave per SIMD nothing hides the softmax and LDS latency between the two MFMA phases.
  return launch_mask<D, 2>(p, stream);
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream) {
  if (p.num_seqs <= 0 || p.max_query_len <= 0) return hipSuccess;
  return p.head_size == 64 ? launch_rows<64>(p, stream) : launch_rows<128>(p, stream);
}

}  // namespace attn
