// Device-side helpers: number formats, FP4 block dot products, wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe_fp4 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ue8m0 scale byte -> 2^(e - 127) in fp32 (2^-127 is an fp32 subnormal; e = 255 is NaN).
__device__ __forceinline__ float ue8m0_to_f32(uint32_t e) {
  const float s = __builtin_amdgcn_ldexpf(1.0f, (int)e - 127);
  return e == 255u ? __builtin_nanf("") : s;
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) {
  return __builtin_bit_cast(bf16x2_t, v);
}

// Dot product of one 32-element FP4 block (16 bytes: byte b holds elements 2b (low nibble)
// and 2b+1 (high nibble)) with 32 bf16 activations (64 bytes, natural order), unscaled.
// Each byte becomes an exact bf16 pair (the conversion's scale operand is 1.0); v_dot2
// multiplies it with the matching activation pair and accumulates in fp32.
__device__ __forceinline__ float fp4_block_dot(const uint4 c, const uint4 a0, const uint4 a1,
                                               const uint4 a2, const uint4 a3) {
  float s0 = 0.f, s1 = 0.f;
#define MOE_FP4_DOT_WORD(W, A)                                                              \
  s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(W, 1.0f, 0), \
                                       as_bf16x2((A).x), s0, false);                        \
  s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(W, 1.0f, 1), \
                                       as_bf16x2((A).y), s1, false);                        \
  s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(W, 1.0f, 2), \
                                       as_bf16x2((A).z), s0, false);                        \
  s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(W, 1.0f, 3), \
                                       as_bf16x2((A).w), s1, false);
  MOE_FP4_DOT_WORD(c.x, a0)
  MOE_FP4_DOT_WORD(c.y, a1)
  MOE_FP4_DOT_WORD(c.z, a2)
  MOE_FP4_DOT_WORD(c.w, a3)
#undef MOE_FP4_DOT_WORD
  return s0 + s1;
}

// Sum over groups of LPR consecutive lanes (LPR a power of two <= 64); every lane of the
// group ends with the group sum. All 64 lanes must execute this call.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

template <int LPR>
__device__ __forceinline__ double group_sum_f64(double v) {
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ float silu_f32(float z) {
  return z / (1.0f + __expf(-z));
}

}  // namespace moe_fp4
