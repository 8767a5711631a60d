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

// One workgroup per row: the shared row helpers (norm_row_add, norm_row_inv,
// norm_row_pack8) give the arithmetic; r_out may be r_in (each thread rewrites only the
// elements it read).
template <int NIT>
__global__ __launch_bounds__(kNormThreads) void residual_rmsnorm_kernel(const float* r_in,
                                                                         const uint16_t* __restrict__ y,
                                                                         float* r_out,
                                                                         uint16_t* __restrict__ x, int H,
                                                                         float eps) {
  static_assert(kNormThreads == kNormRowThreads, "row helpers assume 256 threads");
  __shared__ double part[kNormThreads / 64];
  const long base = (long)blockIdx.x * H;
  const int tid = threadIdx.x;
  float4 ra[NIT], rb[NIT];
  double ss = norm_row_add<NIT>(r_in + base, y + base, H, tid, ra, rb);
  ss = wave_sum_f64(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  const double inv = norm_row_inv(part, H, eps);
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int i0 = 8 * (tid + it * kNormThreads);
    if (i0 < H) {
      *reinterpret_cast<float4*>(r_out + base + i0) = ra[it];
      *reinterpret_cast<float4*>(r_out + base + i0 + 4) = rb[it];
      *reinterpret_cast<uint4*>(x + base + i0) = norm_row_pack8(ra[it], rb[it], inv);
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

hipError_t launch_residual_rmsnorm(const float* r_in, const uint16_t* y, float* r_out, uint16_t* x,
                                   int T, int hidden, float eps, hipStream_t s) {
  if (hidden % 8 != 0 || hidden > 8 * 8 * kNormThreads) return hipErrorInvalidValue;
  const int nit = (hidden + 8 * kNormThreads - 1) / (8 * kNormThreads);
#define MOE_FP4_NORM_LAUNCH(N)                                                                    \
  return launch_kernel(kKindNorm, residual_rmsnorm_kernel<N>, dim3((unsigned)T), dim3(kNormThreads), \
                       0, s, r_in, y, r_out, x, hidden, eps)
  if (nit <= 1) MOE_FP4_NORM_LAUNCH(1);
  if (nit <= 2) MOE_FP4_NORM_LAUNCH(2);
  if (nit <= 4) MOE_FP4_NORM_LAUNCH(4);
  MOE_FP4_NORM_LAUNCH(8);
#undef MOE_FP4_NORM_LAUNCH
}

}  // namespace moe_fp4
