// Prefill attention kernel, bf16 in / fp32 accumulate, for gfx950.
//
// Method (vLLM FlashAttention page, sections "들어가며" and "논문 핵심 내용"): Q, K and V are
// brought on chip tile by tile, the softmax is carried online with a running max and a running
// sum, and only the final rows (plus their log-sum-exp) are written, so no score matrix ever
// reaches HBM. K/V rows are read through the block table from the paged cache of the
// FlashAttentionBackend section; GQA follows num_queries_per_kv of the FlashAttentionImpl
// section; causal and sliding-window masks follow the RBLN "Attention 모드" page.
//
// Work split: one workgroup = 4 waves = 128 query rows of one (request, q head); each wave owns
// 32 rows (two 16-row MFMA columns). KV is walked in 64-key tiles. Per tile:
//   * all 256 threads gather the K and V rows (16-byte loads, one block-table lookup per row)
//     into row-major LDS tiles; the next tile's loads are issued before this tile's math;
//   * S^T = K . Q^T on v_mfma_f32_16x16x32_bf16 (K from LDS as the A operand, Q^T held in
//     registers as the B operand), so each lane holds 4 keys of one query: the row max and row
//     sum need only the 4 lanes of a column (v_permlane16/32_swap);
//   * P^T stays in registers and is already in the B-operand layout of the next MFMA;
//   * O^T += V^T . P^T, with V^T read straight from the row-major V tile by
//     ds_read_b64_tr_b16, so no transpose pass is needed;
//   * each lane owns one query column of O^T, so the online-softmax rescale is lane-local.
#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kBR = 128;      // query rows per workgroup
constexpr int kBC = 64;       // keys per KV tile
constexpr int kWaves = 4;
constexpr int kRowsPerWave = kBR / kWaves;   // 32
constexpr int kQS = kRowsPerWave / 16;       // 16-row MFMA columns per wave

template <int D, bool CAUSAL, bool WINDOW>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(const PrefillParams p) {
  constexpr int RS = D + 16;          // LDS row stride in bf16 (padding against bank conflicts)
  constexpr int KC = D / 32;          // k-chunks of the QK^T contraction
  constexpr int DC = D / 16;          // 16-wide d chunks of O^T
  constexpr int TPR = D / 8;          // threads per K/V row in the gather (16 bytes each)
  constexpr int RPP = 256 / TPR;      // rows per gather pass
  constexpr int NP = kBC / RPP;       // gather passes per tile

  __shared__ __attribute__((aligned(16))) __bf16 sK[kBC * RS];
  __shared__ __attribute__((aligned(16))) __bf16 sV[kBC * RS];

  const int r = p.seq_begin + blockIdx.z;
  const int h = blockIdx.y;
  const int qt = gridDim.x - 1 - blockIdx.x;   // longest (causal) tiles are dispatched first
  const int q_start = p.qsl[r];
  const int ql = p.qsl[r + 1] - q_start;
  if (qt * kBR >= ql) return;
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
  bf16x8 qf[kQS][KC];
  const int wrow0 = qt * kBR + w * kRowsPerWave;        // first query row of this wave
#pragma unroll
  for (int s = 0; s < kQS; ++s) {
    const int row = wrow0 + s * 16 + li;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if (row < ql) {
        qf[s][c] = *reinterpret_cast<const bf16x8*>(q + (int64_t)(q_start + row) * row_stride +
                                                    (int64_t)h * D + 32 * c + 8 * G);
      } else {
        qf[s][c] = bf16x8{};
      }
    }
  }

  // ---- KV range of the workgroup and of this wave
  const int row_lo = qt * kBR;
  const int row_hi = min(ql, row_lo + kBR) - 1;
  const int kv_hi = CAUSAL ? min(sl, cl + row_hi + 1) : sl;
  const int kv_lo = WINDOW ? max(0, cl + row_lo - p.window + 1) : 0;
  const int t_begin = kv_lo / kBC;
  const int t_end = (kv_hi + kBC - 1) / kBC;
  const int w_row_lo = wrow0;
  const int w_row_hi = min(ql, wrow0 + kRowsPerWave) - 1;
  const bool wave_active = w_row_lo <= w_row_hi;
  const int w_kv_hi = CAUSAL ? min(sl, cl + w_row_hi + 1) : sl;
  const int w_kv_lo = WINDOW ? max(0, cl + w_row_lo - p.window + 1) : 0;

  // ---- gather assignment: thread -> (row in pass, 16-byte chunk)
  const int g_row = tid / TPR;
  const int g_chunk = tid % TPR;
  u32x4 kreg[NP], vreg[NP];
  auto gather = [&](int tile) {
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int key = tile * kBC + pp * RPP + g_row;
      if (key < sl) {
        const int32_t blk = bt[key / p.block_size];
        const int64_t off = paged_row(blk, key % p.block_size, kvh, p.block_size,
                                      p.num_kv_heads, D) + g_chunk * 8;
        kreg[pp] = *reinterpret_cast<const u32x4*>(kcache + off);
        vreg[pp] = *reinterpret_cast<const u32x4*>(vcache + off);
      } else {
        kreg[pp] = u32x4{0, 0, 0, 0};   // keys past seq_len: zero, never NaN from stale slots
        vreg[pp] = u32x4{0, 0, 0, 0};
      }
    }
  };

  const float c_log2 = p.scale * kLog2e;
  float m_run[kQS], l_run[kQS];
  floatx4 o[kQS][DC];
#pragma unroll
  for (int s = 0; s < kQS; ++s) {
    m_run[s] = -INFINITY;
    l_run[s] = 0.f;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) o[s][dc] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  if (t_begin < t_end) gather(t_begin);
  for (int t = t_begin; t < t_end; ++t) {
    __syncthreads();   // every wave is done reading the previous tile
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      *reinterpret_cast<u32x4*>(&sK[(pp * RPP + g_row) * RS + g_chunk * 8]) = kreg[pp];
      *reinterpret_cast<u32x4*>(&sV[(pp * RPP + g_row) * RS + g_chunk * 8]) = vreg[pp];
    }
    __syncthreads();
    if (t + 1 < t_end) gather(t + 1);

    const int kb = t * kBC;
    if (!wave_active || kb >= w_kv_hi || kb + kBC <= w_kv_lo) continue;

    // S^T tiles: s[s][kt] holds keys kb + 16kt + 4G + e of query column li
    floatx4 sc[kQS][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      bf16x8 kf[KC];
#pragma unroll
      for (int c = 0; c < KC; ++c)
        kf[c] = *reinterpret_cast<const bf16x8*>(&sK[(kt * 16 + li) * RS + 32 * c + 8 * G]);
#pragma unroll
      for (int s = 0; s < kQS; ++s) {
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
      for (int s = 0; s < kQS; ++s) {
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

    // online softmax, one query column per lane
#pragma unroll
    for (int s = 0; s < kQS; ++s) {
      float mx = sc[s][0][0];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sc[s][kt][e]);
      mx = column_max(mx);
      const float m_new = fmaxf(m_run[s], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2((m_run[s] - m_use) * c_log2);
      const float mc = m_use * c_log2;
      float lsum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pv = fast_exp2(fmaf(sc[s][kt][e], c_log2, -mc));
          sc[s][kt][e] = pv;
          lsum += pv;
        }
      l_run[s] = l_run[s] * alpha + lsum;
      m_run[s] = m_new;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) o[s][dc] *= alpha;
    }

    // O^T += V^T . P^T over two 32-key halves
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
      bf16x8 pb[kQS];
#pragma unroll
      for (int s = 0; s < kQS; ++s) pb[s] = pack_bf16x8(sc[s][2 * hk], sc[s][2 * hk + 1]);
      const int r0 = 32 * hk + 4 * G + li / 4;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const int col = 16 * dc + 4 * (li % 4);
        const bf16x8 va = concat(lds_read_tr16(&sV[r0 * RS + col]),
                                 lds_read_tr16(&sV[(r0 + 16) * RS + col]));
#pragma unroll
        for (int s = 0; s < kQS; ++s) o[s][dc] = mfma16x16x32(va, pb[s], o[s][dc]);
      }
    }
  }

  // ---- epilogue: O / l and lse = scale * m + ln l
  __bf16* __restrict__ out = static_cast<__bf16*>(p.out);
#pragma unroll
  for (int s = 0; s < kQS; ++s) {
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
          l_tot > 0.f ? p.scale * m_run[s] + __logf(l_tot) : -INFINITY;
    }
  }
}

template <int D, bool CAUSAL, bool WINDOW>
hipError_t launch(const PrefillParams& p, hipStream_t stream) {
  const dim3 grid((p.max_query_len + kBR - 1) / kBR, p.num_heads, p.num_seqs);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, WINDOW>), grid, dim3(256), 0, stream, p);
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
