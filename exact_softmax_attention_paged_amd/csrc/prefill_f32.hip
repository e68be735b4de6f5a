// Prefill attention kernel for float32 inputs (fp32 MFMA), for gfx950.
//
// Same method and masks as the bf16 kernel (tiles on chip, online softmax, paged K/V through
// the block table; vLLM FlashAttention page and RBLN "Attention 모드" page), built on
// v_mfma_f32_16x16x4_f32 so that float32 inputs are never rounded to bf16.
//
// Work split: one workgroup = 4 waves = 64 query rows of one (request, q head); each wave owns
// one 16-row MFMA column. KV is walked in 64-key tiles staged in LDS.
//   * S^T = K . Q^T: the k index of every 16x16x4 step is the lane group G; step c covers
//     d = (D/4) G + c, so K and Q^T are read as contiguous runs of D/4 floats per lane;
//   * the S^T result already holds P^T in the B-operand layout of the PV step: P^T element
//     (key 16 kt + 4 G + e, query li) sits in register e of lane (G, li);
//   * O^T += V^T . P^T with one float of V per lane and step (row-major V tile in LDS).
#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kBR = 64;
constexpr int kBC = 64;

template <int D, bool CAUSAL, bool WINDOW>
__global__ __launch_bounds__(256, 1) void prefill_f32_kernel(const PrefillParams p) {
  constexpr int RS = D + 4;         // LDS row stride in floats
  constexpr int DQ = D / 4;         // floats of q / k per lane (one k-slot of the MFMA)
  constexpr int DC = D / 16;
  constexpr int TPR = D / 4;        // threads per row in the gather (16 bytes each)
  constexpr int RPP = 256 / TPR;
  constexpr int NP = kBC / RPP;

  __shared__ __attribute__((aligned(16))) float sK[kBC * RS];
  __shared__ __attribute__((aligned(16))) float sV[kBC * RS];

  const int r = p.seq_begin + blockIdx.z;
  const int h = blockIdx.y;
  const int qt = gridDim.x - 1 - blockIdx.x;
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

  const float* __restrict__ q = static_cast<const float*>(p.q);
  const float* __restrict__ kcache = static_cast<const float*>(p.kv);
  const float* __restrict__ vcache = kcache + p.v_offset;
  const int32_t* __restrict__ bt = p.block_table + (int64_t)r * p.max_blocks;
  const int64_t row_stride = (int64_t)p.num_heads * D;

  const int wrow0 = qt * kBR + w * 16;
  const int my_row = wrow0 + li;
  float qf[DQ];
#pragma unroll
  for (int c = 0; c < DQ; c += 4) {
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (my_row < ql)
      v = *reinterpret_cast<const floatx4*>(q + (int64_t)(q_start + my_row) * row_stride +
                                            (int64_t)h * D + DQ * G + c);
    qf[c] = v[0]; qf[c + 1] = v[1]; qf[c + 2] = v[2]; qf[c + 3] = v[3];
  }

  const int row_lo = qt * kBR;
  const int row_hi = min(ql, row_lo + kBR) - 1;
  const int kv_hi = CAUSAL ? min(sl, cl + row_hi + 1) : sl;
  const int kv_lo = WINDOW ? max(0, cl + row_lo - p.window + 1) : 0;
  const int t_begin = kv_lo / kBC;
  const int t_end = (kv_hi + kBC - 1) / kBC;
  const int w_row_lo = wrow0;
  const int w_row_hi = min(ql, wrow0 + 16) - 1;
  const bool wave_active = w_row_lo <= w_row_hi;
  const int w_kv_hi = CAUSAL ? min(sl, cl + w_row_hi + 1) : sl;
  const int w_kv_lo = WINDOW ? max(0, cl + w_row_lo - p.window + 1) : 0;

  const int g_row = tid / TPR;
  const int g_chunk = tid % TPR;
  floatx4 kreg[NP], vreg[NP];
  auto gather = [&](int tile) {
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int key = tile * kBC + pp * RPP + g_row;
      if (key < sl) {
        const int32_t blk = bt[key / p.block_size];
        const int64_t off = paged_row(blk, key % p.block_size, kvh, p.block_size,
                                      p.num_kv_heads, D) + g_chunk * 4;
        kreg[pp] = *reinterpret_cast<const floatx4*>(kcache + off);
        vreg[pp] = *reinterpret_cast<const floatx4*>(vcache + off);
      } else {
        kreg[pp] = floatx4{0.f, 0.f, 0.f, 0.f};
        vreg[pp] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };

  const float c_log2 = p.scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;
  floatx4 o[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) o[dc] = floatx4{0.f, 0.f, 0.f, 0.f};

  if (t_begin < t_end) gather(t_begin);
  for (int t = t_begin; t < t_end; ++t) {
    __syncthreads();
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      *reinterpret_cast<floatx4*>(&sK[(pp * RPP + g_row) * RS + g_chunk * 4]) = kreg[pp];
      *reinterpret_cast<floatx4*>(&sV[(pp * RPP + g_row) * RS + g_chunk * 4]) = vreg[pp];
    }
    __syncthreads();
    if (t + 1 < t_end) gather(t + 1);

    const int kb = t * kBC;
    if (!wave_active || kb >= w_kv_hi || kb + kBC <= w_kv_lo) continue;

    floatx4 sc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      const float* krow = &sK[(kt * 16 + li) * RS + DQ * G];
#pragma unroll
      for (int c = 0; c < DQ; c += 4) {
        const floatx4 kv4 = *reinterpret_cast<const floatx4*>(krow + c);
        acc = mfma16x16x4f32(kv4[0], qf[c], acc);
        acc = mfma16x16x4f32(kv4[1], qf[c + 1], acc);
        acc = mfma16x16x4f32(kv4[2], qf[c + 2], acc);
        acc = mfma16x16x4f32(kv4[3], qf[c + 3], acc);
      }
      sc[kt] = acc;
    }

    const bool need_mask = (kb + kBC > sl) || (CAUSAL && kb + kBC - 1 > cl + w_row_lo) ||
                           (WINDOW && kb < cl + w_row_hi - p.window + 1);
    if (need_mask) {
      const int pos = cl + my_row;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = kb + kt * 16 + 4 * G + e;
          bool vis = j < sl;
          if (CAUSAL) vis = vis && (j <= pos);
          if (WINDOW) vis = vis && (j >= pos - p.window + 1);
          if (!vis) sc[kt][e] = -INFINITY;
        }
    }

    float mx = sc[0][0];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sc[kt][e]);
    mx = column_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2((m_run - m_use) * c_log2);
    const float mc = m_use * c_log2;
    float lsum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pv = fast_exp2(fmaf(sc[kt][e], c_log2, -mc));
        sc[kt][e] = pv;
        lsum += pv;
      }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) o[dc] *= alpha;

#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float* vrow = &sV[(kt * 16 + 4 * G + e) * RS + li];
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) o[dc] = mfma16x16x4f32(vrow[16 * dc], sc[kt][e], o[dc]);
      }
  }

  const float l_tot = column_sum(l_run);
  if (my_row < ql) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* dst = static_cast<float*>(p.out) + (int64_t)(q_start + my_row) * row_stride +
                 (int64_t)h * D + 4 * G;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      *reinterpret_cast<floatx4*>(dst + 16 * dc) = o[dc] * inv;
    if (p.lse != nullptr && G == 0)
      p.lse[(int64_t)(q_start + my_row) * p.num_heads + h] =
          l_tot > 0.f ? p.scale * m_run + logf(l_tot) : -INFINITY;
  }
}

template <int D, bool CAUSAL, bool WINDOW>
hipError_t launch(const PrefillParams& p, hipStream_t stream) {
  const dim3 grid((p.max_query_len + kBR - 1) / kBR, p.num_heads, p.num_seqs);
  hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL, WINDOW>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mask(const PrefillParams& p, hipStream_t stream) {
  if (p.window > 0) return launch<D, true, true>(p, stream);
  if (p.causal) return launch<D, true, false>(p, stream);
  return launch<D, false, false>(p, stream);
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillParams& p, hipStream_t stream) {
  if (p.num_seqs <= 0 || p.max_query_len <= 0) return hipSuccess;
  return p.head_size == 64 ? launch_mask<64>(p, stream) : launch_mask<128>(p, stream);
}

}  // namespace attn
