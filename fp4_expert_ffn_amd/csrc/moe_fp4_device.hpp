// Device-side helpers: number formats, wavefront reductions, the router selection and the
// residual + RMSNorm row helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
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

// fp64 value moved across lanes by a DPP pattern (both 32-bit halves alike).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)b, CTRL, 0xF, 0xF, false);
  const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Sum over the 64 lanes of a wavefront (all lanes active); every lane gets the same sum.
// Pairs of lanes add each other's partial sums: DPP inside 16-lane rows (quad swaps, then
// the 8- and 16-lane mirrors), then gfx950's lane swaps across rows. Partners add the same
// two operands (a + b and b + a are equal in IEEE arithmetic), so all lanes hold identical
// bits, and the pairing is the same on every call.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f64<0x141>(v);  // row_half_mirror
  v += dpp_f64<0x140>(v);  // row_mirror
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const auto l32 = __builtin_amdgcn_permlane32_swap((unsigned)b, (unsigned)b, false, false);
  const auto h32 = __builtin_amdgcn_permlane32_swap((unsigned)(b >> 32), (unsigned)(b >> 32), false, false);
  v = __longlong_as_double((long long)(((unsigned long long)(unsigned)h32[0] << 32) | (unsigned)l32[0])) +
      __longlong_as_double((long long)(((unsigned long long)(unsigned)h32[1] << 32) | (unsigned)l32[1]));
  const unsigned long long c = (unsigned long long)__double_as_longlong(v);
  const auto l16 = __builtin_amdgcn_permlane16_swap((unsigned)c, (unsigned)c, false, false);
  const auto h16 = __builtin_amdgcn_permlane16_swap((unsigned)(c >> 32), (unsigned)(c >> 32), false, false);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)h16[0] << 32) | (unsigned)l16[0])) +
         __longlong_as_double((long long)(((unsigned long long)(unsigned)h16[1] << 32) | (unsigned)l16[1]));
}

// Wave-wide maximum of a uint32 (all 64 lanes active): a DPP butterfly inside each row of
// 16 lanes, then two lane swaps across rows. Every lane gets the result.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  // every lane now holds its 16-lane row's maximum; gfx950's lane swaps combine the rows
  // in vector registers (rows 2, 3 against rows 0, 1, then odd against even rows), so the
  // result reaches every lane without scalar round trips
  const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = max((uint32_t)h[0], (uint32_t)h[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max((uint32_t)q[0], (uint32_t)q[1]);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return ~wave_max_u32(~v); }

// Residual add and RMS normalisation of one row of H elements (H % 8 == 0), shared by the
// standalone norm kernel and the router kernel that normalises its own input, so both give
// identical bits. Thread t of the kNormRowThreads owns the NIT groups of 8 consecutive
// elements starting at 8 (t + kNormRowThreads it): norm_row_add loads them (all loads
// issued before any use), adds y to r in fp32 and returns the thread's fp64 sum of squares
// in a fixed order; the caller reduces it over the four wavefronts in wave order, and
// norm_row_pack8 rounds r * inv of one group to bf16.
constexpr int kNormRowThreads = 256;

template <int NIT>
__device__ __forceinline__ double norm_row_add(const float* __restrict__ r, const uint16_t* __restrict__ y,
                                               int H, int t, float4 (&ra)[NIT], float4 (&rb)[NIT]) {
  uint4 yv[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int i0 = 8 * (t + it * kNormRowThreads);
    ra[it] = rb[it] = make_float4(0.f, 0.f, 0.f, 0.f);
    yv[it] = make_uint4(0, 0, 0, 0);
    if (i0 < H) {
      ra[it] = *reinterpret_cast<const float4*>(r + i0);
      rb[it] = *reinterpret_cast<const float4*>(r + i0 + 4);
      yv[it] = *reinterpret_cast<const uint4*>(y + i0);
    }
  }
  double ss = 0.0;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    ra[it].x += bf16_bits_to_f32(yv[it].x & 0xffffu);
    ra[it].y += bf16_bits_to_f32(yv[it].x >> 16);
    ra[it].z += bf16_bits_to_f32(yv[it].y & 0xffffu);
    ra[it].w += bf16_bits_to_f32(yv[it].y >> 16);
    rb[it].x += bf16_bits_to_f32(yv[it].z & 0xffffu);
    rb[it].y += bf16_bits_to_f32(yv[it].z >> 16);
    rb[it].z += bf16_bits_to_f32(yv[it].w & 0xffffu);
    rb[it].w += bf16_bits_to_f32(yv[it].w >> 16);
    ss += (double)ra[it].x * ra[it].x + (double)ra[it].y * ra[it].y +
          (double)ra[it].z * ra[it].z + (double)ra[it].w * ra[it].w +
          (double)rb[it].x * rb[it].x + (double)rb[it].y * rb[it].y +
          (double)rb[it].z * rb[it].z + (double)rb[it].w * rb[it].w;
  }
  return ss;
}

__device__ __forceinline__ uint4 norm_row_pack8(const float4& a, const float4& b, double inv) {
  const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = (uint32_t)f32_to_bf16_rne((float)((double)f[2 * q] * inv)) |
           ((uint32_t)f32_to_bf16_rne((float)((double)f[2 * q + 1] * inv)) << 16);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// inv = 1 / sqrt(mean of squares + eps) from the four wavefronts' partial sums, in order.
__device__ __forceinline__ double norm_row_inv(const double* part, int H, float eps) {
  double tot = 0.0;
#pragma unroll
  for (int w = 0; w < kNormRowThreads / 64; ++w) tot += part[w];
  return 1.0 / sqrt(tot / H + (double)eps);
}

// Order-preserving map of an fp64 value to uint64 (larger value -> larger key; -0 and +0
// map to the same key). NaN is not ordered meaningfully.
__device__ __forceinline__ uint64_t f64_order_key(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v + 0.0);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ double f64_from_order_key(uint64_t k) {
  const uint64_t u = (k >> 63) ? (k & 0x7fffffffffffffffull) : ~k;
  return __longlong_as_double((long long)u);
}

// Softmax over the k selected logits v[0..k-1] (v[0] the largest, the same v on every
// lane of the wavefront), fp64, summed in slot order, rounded to fp32: the one definition
// of the router weights. Lane j < k evaluates slot j's exponential and quotient, so the
// wavefront pays for one exp and one division instead of k of each; on return every lane
// holds all k weights.
__device__ __forceinline__ void topk_softmax_weights(const double (&v)[8], int k, int lane,
                                                     float (&w)[8]) {
  double vl = v[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) vl = (lane == j) ? v[j] : vl;
  const double ex = (lane < k) ? exp(vl - v[0]) : 0.0;
  const uint64_t exb = (uint64_t)__double_as_longlong(ex);
  double sum = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < k) {
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)exb, j);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(exb >> 32), j);
      sum += __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
    }
  }
  const float wl = (float)(ex / sum);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    w[j] = (j < k) ? __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wl), j)) : 0.f;
}

// (key, id) order of the selection: larger key first, equal keys by smaller id.
__device__ __forceinline__ bool topk_before(uint64_t ka, int ia, uint64_t kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// Top-k of one row of E logits by a whole wavefront (all 64 lanes active, wave-uniform
// arguments). Lane l holds the order keys of logits l, l + 64, ... (at most PER per lane)
// and sorts them once, best first, with an odd-even transposition network. Each of the k
// rounds then looks only at the lanes' heads: a DPP maximum of the heads' high key words;
// when a single lane holds it (the usual case) that lane's head is the winner, otherwise
// the low words and then the ids decide among the tied lanes. The winning lane shifts its
// list by one. On return every lane holds ids[j] (descending logit, ties by ascending
// id) and w[j] = softmax over the k selected logits (fp64, rounded to fp32), for j < k.
template <int PER, bool WEIGHTS = true, typename V>
__device__ __forceinline__ void wave_topk(const V* __restrict__ row, int E, int k, int lane,
                                          int (&ids)[8], float (&w)[8]) {
  uint64_t key[PER];
  int kid[PER];
  double lv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) lv[i] = (double)row[min(lane + i * 64, E - 1)];  // clamped
  // an empty asm that takes each loaded value keeps the loads unconditional (the compiler
  // would otherwise sink each into the branch of its select, waiting after every one), so
  // all PER loads are in flight together
#pragma unroll
  for (int i = 0; i < PER; ++i) __asm__ volatile("" : "+v"(lv[i]));
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + i * 64;
    key[i] = (e < E) ? f64_order_key(lv[i]) : 0ull;  // 0: empty slot
    kid[i] = (e < E) ? e : 0x7fffffff;
  }
#pragma unroll
  for (int pass = 0; pass < PER; ++pass) {
#pragma unroll
    for (int i = pass & 1; i + 1 < PER; i += 2) {
      if (topk_before(key[i + 1], kid[i + 1], key[i], kid[i])) {
        const uint64_t tk = key[i];
        key[i] = key[i + 1];
        key[i + 1] = tk;
        const int ti = kid[i];
        kid[i] = kid[i + 1];
        kid[i + 1] = ti;
      }
    }
  }
  double v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ids[j] = 0;
    v[j] = 0.0;
    if (j < k) {
      const uint32_t hk = (uint32_t)(key[0] >> 32);
      const uint32_t hi = wave_max_u32(hk);
      const unsigned long long tied = __ballot(hk == hi);
      int wl;
      uint64_t mk;
      if (__popcll(tied) == 1) {  // wave-uniform
        wl = __ffsll((long long)tied) - 1;
        mk = ((uint64_t)hi << 32) | (uint32_t)__builtin_amdgcn_readlane((uint32_t)key[0], wl);
      } else {
        const uint32_t lo = wave_max_u32(hk == hi ? (uint32_t)key[0] : 0u);
        mk = ((uint64_t)hi << 32) | lo;
        const uint32_t mid = wave_min_u32(key[0] == mk ? (uint32_t)kid[0] : 0xffffffffu);
        wl = (int)(mid & 63u);  // a lane's ids are congruent to the lane mod 64
      }
      ids[j] = __builtin_amdgcn_readlane(kid[0], wl);
      v[j] = f64_from_order_key(mk);
      if (lane == wl) {
#pragma unroll
        for (int i = 0; i + 1 < PER; ++i) {
          key[i] = key[i + 1];
          kid[i] = kid[i + 1];
        }
        key[PER - 1] = 0ull;
        kid[PER - 1] = 0x7fffffff;
      }
    }
  }
  if constexpr (WEIGHTS) {
    topk_softmax_weights(v, k, lane, w);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = 0.f;
  }
}

__device__ __forceinline__ float silu_f32(float z) {
  return z / (1.0f + __expf(-z));
}

}  // namespace moe_fp4
