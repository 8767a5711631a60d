// Measurement kernels for the rooflines' measured peaks (not on the FFN path):
//  - a pure streaming read of a device buffer with the same 16-byte non-temporal loads the
//    expert kernels use, so "fraction of what this chip streams" can be quoted beside the
//    fraction of the published 8 TB/s;
//  - a tight loop of the block-scaled matrix-core operation the grouped GEMM issues
//    (v_mfma_scale_f32_16x16x128_f8f6f4, B in FP4 E2M1, A in FP4 or FP8 E4M3), for the
//    matrix-core peak this chip sustains.
// Both keep their work alive through a data-dependent store to `sink` that practically
// never executes.
#include "moe_fp4_device.hpp"
#include "moe_fp4_internal.hpp"

namespace moe_fp4 {

namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;  // 16-byte loads in flight per lane
constexpr uint32_t kNeverWord = 0x9E3779B9u;

__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Grid-stride over n16 16-byte words; every lane keeps kStreamUnroll loads in flight.
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const uint4* __restrict__ src,
                                                                     size_t n16,
                                                                     uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kStreamThreads;
  size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (size_t)(kStreamUnroll - 1) * stride < n16; i += (size_t)kStreamUnroll * stride) {
    uint4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = ld_nt(src + i + (size_t)u * stride);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = ld_nt(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == kNeverWord) *sink = acc;
}

// Eight independent accumulation chains per wavefront, operands fixed in registers (the
// operation's timing does not depend on the values). FMT_A: 4 = FP4 E2M1, 0 = FP8 E4M3.
constexpr int kMfmaChains = 8;

template <int FMT_A>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int seed = lane + 64 * (int)blockIdx.x;
  // bytes below 0x40: finite in every format (FP8 E4M3 NaN is 0x7F / 0xFF)
  const int word = (int)(((uint32_t)seed * 0x01010101u) & 0x3F3F3F3Fu);
  const i32x8_t a = {word, word ^ 0x01010101, word ^ 0x02020202, word ^ 0x03030303,
                     word ^ 0x04040404, word ^ 0x05050505, word ^ 0x06060606, word ^ 0x07070707};
  const i32x8_t b = {word ^ 0x10101010, word ^ 0x11111111, word ^ 0x12121212, word ^ 0x13131313,
                     0, 0, 0, 0};
  const int sa = 120 + (lane & 7), sb = 120 + ((lane >> 3) & 7);
  // named accumulators: an array carried around the loop is shuffled between registers
  f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
  static_assert(kMfmaChains == 8, "eight chains");
  for (int it = 0; it < iters; ++it) {
#define MOE_FP4_PROBE_MFMA(C) C = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, C, FMT_A, 4, 0, sa, 0, sb)
    MOE_FP4_PROBE_MFMA(c0);
    MOE_FP4_PROBE_MFMA(c1);
    MOE_FP4_PROBE_MFMA(c2);
    MOE_FP4_PROBE_MFMA(c3);
    MOE_FP4_PROBE_MFMA(c4);
    MOE_FP4_PROBE_MFMA(c5);
    MOE_FP4_PROBE_MFMA(c6);
    MOE_FP4_PROBE_MFMA(c7);
#undef MOE_FP4_PROBE_MFMA
  }
  const f32x4_t t = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
  const float s = (t[0] + t[1]) + (t[2] + t[3]);
  if (__float_as_uint(s) == kNeverWord) *sink = __float_as_uint(s);
}

}  // namespace

hipError_t launch_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
  const size_t n16 = bytes / 16;
  const size_t per_wg = (size_t)kStreamThreads * kStreamUnroll;
  const size_t want = (n16 + per_wg - 1) / per_wg;
  const unsigned grid = (unsigned)(want < 2048 ? (want > 0 ? want : 1) : 2048);
  return launch_kernel(kKindProbeStream, stream_read_kernel, dim3(grid), dim3(kStreamThreads), 0, s,
                       static_cast<const uint4*>(src), n16, sink);
}

hipError_t launch_probe_mfma_loop(int fmt_a, int n_workgroups, int iters, uint32_t* sink,
                                  hipStream_t s) {
  if (fmt_a == 4)
    return launch_kernel(kKindProbeMfma, mfma_loop_kernel<4>, dim3((unsigned)n_workgroups),
                         dim3(256), 0, s, iters, sink);
  return launch_kernel(kKindProbeMfma, mfma_loop_kernel<0>, dim3((unsigned)n_workgroups), dim3(256),
                       0, s, iters, sink);
}

int probe_mfma_chains() { return kMfmaChains; }

}  // namespace moe_fp4
