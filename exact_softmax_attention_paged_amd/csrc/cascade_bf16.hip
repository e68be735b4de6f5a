// Merge of the key slices of the cascade prefix pass, for gfx950.
//
// When the batch has few query rows, the prefix pass splits the shared prefix's keys into
// slices that run as separate workgroups (so the launch fills the chip); each slice leaves a
// partial result (normalised O and log-sum-exp) per (token, q head). They are combined the
// way partial softmax results over disjoint key sets combine (RBLN "Attention 모드" page,
// Overview: partitions merged by online softmax): L = ln sum_z exp(lse_z),
// O = sum_z exp(lse_z - L) O_z. The result is the prefix partial that the suffix pass starts
// from ("[vLLM] FlashAttention" page, section on cascade attention).
#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

// one wave per (token, head) row; 4 rows per workgroup
template <int D>
__global__ __launch_bounds__(256) void prefix_slices_merge_kernel(const PrefixMergeParams p) {
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (row >= p.rows) return;
  const int lane = threadIdx.x % kWave;
  float M = -INFINITY;
  for (int z = lane; z < p.slices; z += kWave) M = fmaxf(M, p.lse_in[z * p.rows + row]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float M_use = (M == -INFINITY) ? 0.f : M;
  float S = 0.f;
  for (int z = lane; z < p.slices; z += kWave)
    S += fast_exp2((p.lse_in[z * p.rows + row] - M_use) * kLog2e);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) S += __shfl_xor(S, off);
  const float L = S > 0.f ? M_use + __logf(S) : -INFINITY;
  constexpr int DPL = D / kWave;
  float acc[DPL];
#pragma unroll
  for (int x = 0; x < DPL; ++x) acc[x] = 0.f;
  if (S > 0.f) {
    for (int z = 0; z < p.slices; ++z) {
      const float wgt = fast_exp2((p.lse_in[z * p.rows + row] - L) * kLog2e);
      const float* src = p.o_in + (z * p.rows + row) * D;
#pragma unroll
      for (int x = 0; x < DPL; ++x) acc[x] += wgt * src[lane + kWave * x];
    }
  }
  float* dst = p.o_out + row * D;
#pragma unroll
  for (int x = 0; x < DPL; ++x) dst[lane + kWave * x] = acc[x];
  if (lane == 0) p.lse_out[row] = L;
}

}  // namespace

hipError_t launch_prefix_slices_merge(const PrefixMergeParams& p, int head_size,
                                      hipStream_t stream) {
  if (p.rows <= 0 || p.slices <= 1) return hipSuccess;
  const dim3 grid((unsigned)((p.rows + 3) / 4));
  if (head_size == 64)
    hipLaunchKernelGGL(prefix_slices_merge_kernel<64>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(prefix_slices_merge_kernel<128>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
