// Residual add and RMS normalisation between chained MoE layers (a harness step for the
// multi-layer decode workload; RMSNorm is one of the per-layer kernels the pages list among
// the small launches of a decode step, [A100-FP4], section 然后又发现每 token 启动 2000 次内核).
//   residual_init:    r = x (bf16 -> fp32)
//   residual_rmsnorm: r = r + y (fp32), x = bf16(r / sqrt(mean(r^2) + eps)), unit gain.
// One workgroup per token; the mean of squares is accumulated in fp64. hidden must be a
// multiple of 8 and at most 16384.
#include "moe_fp4_device.hpp"
#include "moe_fp4_internal.hpp"

namespace moe_fp4 {

namespace {

constexpr int kNormThreads = 256;

__global__ __launch_bounds__(kNormThreads) void residual_init_kernel(const uint16_t* __restrict__ x,
                                                                      float* __restrict__ r, long n) {
  for (long i = (long)blockIdx.x * kNormThreads + threadIdx.x; i < n; i += (long)gridDim.x * kNormThreads)
    r[i] = bf16_bits_to_f32(x[i]);
}

// Thread t owns NIT groups of 8 consecutive elements (H % 8 == 0, H <= NIT * 8 * 256): all
// of its r and y loads are issued before any use, the sum of squares is reduced across the
// workgroup in a fixed order, and the normalised values are stored from registers.
template <int NIT>
__global__ __launch_bounds__(kNormThreads) void residual_rmsnorm_kernel(float* __restrict__ r,
                                                                         const uint16_t* __restrict__ y,
                                                                         uint16_t* __restrict__ x, int H,
                                                                         float eps) {
  __shared__ double part[kNormThreads / 64];
  const long base = (long)blockIdx.x * H;
  const int tid = threadIdx.x;
  float4 ra[NIT], rb[NIT];
  uint4 yv[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int i0 = 8 * (tid + it * kNormThreads);
    ra[it] = rb[it] = make_float4(0.f, 0.f, 0.f, 0.f);
    yv[it] = make_uint4(0, 0, 0, 0);
    if (i0 < H) {
      ra[it] = *reinterpret_cast<const float4*>(r + base + i0);
      rb[it] = *reinterpret_cast<const float4*>(r + base + i0 + 4);
      yv[it] = *reinterpret_cast<const uint4*>(y + base + i0);
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
  ss = wave_sum_f64(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int w = 0; w < kNormThreads / 64; ++w) tot += part[w];  // fixed order
  const double inv = 1.0 / sqrt(tot / H + (double)eps);
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int i0 = 8 * (tid + it * kNormThreads);
    if (i0 < H) {
      *reinterpret_cast<float4*>(r + base + i0) = ra[it];
      *reinterpret_cast<float4*>(r + base + i0 + 4) = rb[it];
      const float f[8] = {ra[it].x, ra[it].y, ra[it].z, ra[it].w, rb[it].x, rb[it].y, rb[it].z, rb[it].w};
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = (uint32_t)f32_to_bf16_rne((float)((double)f[2 * q] * inv)) |
               ((uint32_t)f32_to_bf16_rne((float)((double)f[2 * q + 1] * inv)) << 16);
      *reinterpret_cast<uint4*>(x + base + i0) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

}  // namespace

hipError_t launch_residual_init(const uint16_t* x, float* r, int T, int hidden, hipStream_t s) {
  const long n = (long)T * hidden;
  long blocks = (n + kNormThreads - 1) / kNormThreads;
  if (blocks > 65536) blocks = 65536;
  return launch_kernel(kKindNorm, residual_init_kernel, dim3((unsigned)blocks), dim3(kNormThreads), 0,
                       s, x, r, n);
}

hipError_t launch_residual_rmsnorm(float* r, const uint16_t* y, uint16_t* x, int T, int hidden,
                                   float eps, hipStream_t s) {
  if (hidden % 8 != 0 || hidden > 8 * 8 * kNormThreads) return hipErrorInvalidValue;
  const int nit = (hidden + 8 * kNormThreads - 1) / (8 * kNormThreads);
#define MOE_FP4_NORM_LAUNCH(N)                                                                    \
  return launch_kernel(kKindNorm, residual_rmsnorm_kernel<N>, dim3((unsigned)T), dim3(kNormThreads), \
                       0, s, r, y, x, hidden, eps)
  if (nit <= 1) MOE_FP4_NORM_LAUNCH(1);
  if (nit <= 2) MOE_FP4_NORM_LAUNCH(2);
  if (nit <= 4) MOE_FP4_NORM_LAUNCH(4);
  MOE_FP4_NORM_LAUNCH(8);
#undef MOE_FP4_NORM_LAUNCH
}

}  // namespace moe_fp4
