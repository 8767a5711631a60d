// Shared pieces of the FP4 weight-streaming matrix-vector kernels (decode and small-M
// paths): the gate/up launch shape, the weight and scale loads, and the in-register FP4 ->
// bf16 conversion that feeds v_mfma_f32_16x16x32_bf16. Everything has internal linkage, so
// each translation unit that includes this gets its own copy.
#pragma once

#include "moe_fp4_device.hpp"

namespace moe_fp4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Launch shapes, tuned by measurement on MI355X; overridable at build time.
#ifndef MOE_FP4_GU_WAVES
#define MOE_FP4_GU_WAVES 4      // wavefronts per gate/up tile (split of K)
#endif
#ifndef MOE_FP4_GU_BATCH
#define MOE_FP4_GU_BATCH 4      // 128-element chunks loaded per wave before use
#endif
#ifndef MOE_FP4_GU_MIN_WAVES
#define MOE_FP4_GU_MIN_WAVES 5  // wavefronts per SIMD the gate/up kernel must allow
#endif

constexpr int kGUWaves = MOE_FP4_GU_WAVES;
constexpr int kGUThreads = kGUWaves * 64;
constexpr int kGUBatch = MOE_FP4_GU_BATCH;
constexpr int kTile = 16;  // weight rows per tile (MFMA N)

// Weight streams are read once per call: non-temporal loads keep them from displacing
// the small reused data (activations, h) in the caches.
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Scale bytes: ordinary cached loads (neighbouring lanes read neighbouring bytes of one
// cache line in separate instructions; through the cache the line is fetched once).
__device__ __forceinline__ uint32_t ld_scale(const uint8_t* p) { return *p; }

// The scale operand of the FP4 conversion: a float whose exponent field is the ue8m0 byte.
// The conversion reads only that field, as an E8M0 scale (measured on gfx950 for every code
// pair and every byte): it multiplies by 2^(e-127) for every e = 0..254, keeping bf16
// subnormal results (e = 0 and 1), and gives NaN for e = 255, zero codes included. A product
// of magnitude 2^128 or more (e = 253 with |code| >= 4, e = 254 with |code| >= 2) is not
// representable in bf16 and becomes +-inf. Every other result is exact: an E2M1 value times
// a power of two has at most two significant bits.
__device__ __forceinline__ float scale_operand(uint32_t e) { return __uint_as_float(e << 23); }

// Eight FP4 codes (one dword, element 2i in the low nibble of byte i) -> eight bf16 values
// times the block scale.
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16(uint32_t w, float s) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
  return bf16x8_t{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint32_t dword(const uint4& v, int m) {
  return m == 0 ? v.x : m == 1 ? v.y : m == 2 ? v.z : v.w;
}

}  // namespace
}  // namespace moe_fp4
