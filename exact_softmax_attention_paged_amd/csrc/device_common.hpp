// Device helpers shared by the gfx950 attention kernels: MFMA operand types, cross-lane
// reductions, bf16 packing and the paged-cache address arithmetic.
//
// Lane layouts (checked on gfx950 with random integer matrices before use):
//   v_mfma_f32_16x16x32_bf16: lane l = 16*G + i (G = l/16, i = l%16)
//     A (16 x 32): element e of lane l is A[i][8G + e]
//     B (32 x 16): element e of lane l is B[8G + e][i]
//     C (16 x 16): element e of lane l is C[4G + e][i]
//   v_mfma_f32_16x16x4_f32: A[i][G], B[G][i], C[4G + e][i].
//   ds_read_b64_tr_b16: inside each 16-lane group, output lane i element j is element i%4 of
//     the 8 bytes addressed by input lane 4j + i/4. Fed with row addresses of a row-major
//     [key][d] tile, it yields MFMA operands whose k index runs over keys.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

__device__ __forceinline__ floatx4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma16x16x4f32(float a, float b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 2^x on the hardware exp unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over the 4 lanes {i, i+16, i+32, i+48} that share a column of an MFMA result.
// v_permlane16_swap exchanges odd 16-lane rows of one operand with even rows of the other;
// with both operands equal, the two results hold each lane's own value and its xor-16
// partner's. v_permlane32_swap does the same for the two 32-lane halves.
__device__ __forceinline__ float max_xor16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float column_max(float v) {
  return max_xor32(max_xor16(v));
}
__device__ __forceinline__ float column_sum(float v) {
  return add_xor32(add_xor16(v));
}

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

__device__ __forceinline__ bf16x8 pack_bf16x8(const floatx4& lo, const floatx4& hi) {
  bf16x8 r;
  r[0] = to_bf16(lo[0]); r[1] = to_bf16(lo[1]); r[2] = to_bf16(lo[2]); r[3] = to_bf16(lo[3]);
  r[4] = to_bf16(hi[0]); r[5] = to_bf16(hi[1]); r[6] = to_bf16(hi[2]); r[7] = to_bf16(hi[3]);
  return r;
}

// Transposing 8-byte LDS read (see the layout note at the top of this file).
__device__ __forceinline__ bf16x4 lds_read_tr16(const void* lds_ptr) {
  shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4*)(lds_ptr));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 concat(const bf16x4& a, const bf16x4& b) {
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// Element offset of row (block, slot, kv head) inside one half (K or V) of the paged cache
// (2, num_blocks, block_size, num_kv_heads, head_size). 64-bit: caches exceed 2^31 elements.
__device__ __forceinline__ int64_t paged_row(int32_t block, int32_t slot, int32_t kvh,
                                             int32_t block_size, int32_t num_kv_heads,
                                             int32_t head_size) {
  return ((int64_t)block * block_size + slot) * (int64_t)num_kv_heads * head_size +
         (int64_t)kvh * head_size;
}

}  // namespace attn
