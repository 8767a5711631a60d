// Router: logits = W_r x in fp64, then top-k selection and softmax over the selection.
// Ids never leave the device ([8GB-GPU], section 提速之路：v1 到 v4: one host round trip per
// expert on the indices was a measured cost; here there is none).
#include <math.h>

#include "moe_fp4_device.hpp"
#include "moe_fp4_internal.hpp"

namespace moe_fp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// One wave per (token, expert) logit. Each bf16 x bf16 product is exact in fp32 (8-bit
// significands), so converting it to fp64 and summing in fp64 rounds only the sum. Every
// logit is summed in the same lane/step order, so identical router rows give bit-identical
// logits (exact ties stay exact ties).
__global__ __launch_bounds__(kThreads) void router_gemv_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ wr,
                                                               int T, int H, int E,
                                                               double* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const long wave = (long)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (wave >= (long)T * E) return;
  const int t = (int)(wave / E);
  const int e = (int)(wave - (long)t * E);
  const uint4* xv = reinterpret_cast<const uint4*>(x + (size_t)t * H);
  const uint4* wv = reinterpret_cast<const uint4*>(wr + (size_t)e * H);
  const int chunks = H / 8;
  double acc = 0.0;
  for (int c = lane; c < chunks; c += 64) {
    const uint4 a = xv[c];
    const uint4 b = wv[c];
    const uint32_t av[4] = {a.x, a.y, a.z, a.w};
    const uint32_t bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float p0 = bf16_bits_to_f32(av[q] & 0xffffu) * bf16_bits_to_f32(bv[q] & 0xffffu);
      const float p1 = bf16_bits_to_f32(av[q] >> 16) * bf16_bits_to_f32(bv[q] >> 16);
      acc += (double)p0;
      acc += (double)p1;
    }
  }
  acc = group_sum_f64<64>(acc);
  if (lane == 0) logits[(size_t)t * E + e] = acc;
}

// "a before b" in selection order: larger logit first, equal logits by smaller id.
template <typename V>
__device__ __forceinline__ bool better(V va, int ia, V vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// One wave per token. Lane l holds logits l, l + 64, ...; k rounds of a wave-wide
// arg-max, each removing its winner. Weights: softmax over the k chosen logits in fp64.
template <typename V>
__global__ __launch_bounds__(kThreads) void topk_kernel(const V* __restrict__ logits, int T, int E,
                                                        int k, int32_t* __restrict__ ids,
                                                        float* __restrict__ w) {
  constexpr int kPer = kMaxExpertsTopk / 64;
  const int lane = threadIdx.x & 63;
  const long t = (long)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const V* row = logits + (size_t)t * E;
  V v[kPer];
  bool taken[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + i * 64;
    taken[i] = e >= E;
    v[i] = (e < E) ? row[e] : (V)0;
  }
  double sel_v[kMaxK];
  int sel_i[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    sel_v[j] = 0.0;
    sel_i[j] = 0;
  }
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      // lane-local best
      V bv = (V)0;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int e = lane + i * 64;
        if (!taken[i] && (bi == 0x7fffffff || better(v[i], e, bv, bi))) {
          bv = v[i];
          bi = e;
        }
      }
      // wave arg-max
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const V ov = __shfl_xor(bv, m, 64);
        const int oi = __shfl_xor(bi, m, 64);
        if (oi != 0x7fffffff && (bi == 0x7fffffff || better(ov, oi, bv, bi))) {
          bv = ov;
          bi = oi;
        }
      }
      // every lane now holds the winner; its owner marks it taken
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (lane + i * 64 == bi) taken[i] = true;
      sel_v[j] = (double)bv;
      sel_i[j] = bi;
    }
  }
  if (lane == 0) {
    double ex[kMaxK];
    double sum = 0.0;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      ex[j] = (j < k) ? exp(sel_v[j] - sel_v[0]) : 0.0;
      sum += ex[j];
    }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        ids[(size_t)t * k + j] = sel_i[j];
        w[(size_t)t * k + j] = (float)(ex[j] / sum);
      }
    }
  }
}

__global__ __launch_bounds__(1024) void validate_ids_kernel(const int32_t* __restrict__ ids,
                                                           long n, int n_experts,
                                                           int32_t* __restrict__ bad) {
  __shared__ int partial[1024 / 64];
  int cnt = 0;
  for (long i = threadIdx.x; i < n; i += 1024) {
    const int e = ids[i];
    cnt += (e < 0 || e >= n_experts) ? 1 : 0;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) cnt += __shfl_xor(cnt, m, 64);
  if ((threadIdx.x & 63) == 0) partial[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int i = 0; i < 1024 / 64; ++i) s += partial[i];
    *bad = s;
  }
}

}  // namespace

hipError_t launch_router_gemv(const uint16_t* x, const uint16_t* wr, int T, int hidden,
                              int n_experts, double* logits, hipStream_t s) {
  const long waves = (long)T * n_experts;
  const long blocks = (waves + kWaves - 1) / kWaves;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(router_gemv_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, x, wr, T,
                     hidden, n_experts, logits);
  return hipGetLastError();
}

hipError_t launch_topk_f64(const double* logits, int T, int n_experts, int k, int32_t* ids,
                           float* w, hipStream_t s) {
  const long blocks = ((long)T + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(topk_kernel<double>, dim3((unsigned)blocks), dim3(kThreads), 0, s, logits,
                     T, n_experts, k, ids, w);
  return hipGetLastError();
}

hipError_t launch_topk_f32(const float* logits, int T, int n_experts, int k, int32_t* ids,
                           float* w, hipStream_t s) {
  const long blocks = ((long)T + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(topk_kernel<float>, dim3((unsigned)blocks), dim3(kThreads), 0, s, logits,
                     T, n_experts, k, ids, w);
  return hipGetLastError();
}

hipError_t launch_validate_ids(const int32_t* ids, int T, int k, int n_experts, int32_t* bad,
                               hipStream_t s) {
  hipLaunchKernelGGL(validate_ids_kernel, dim3(1), dim3(1024), 0, s, ids, (long)T * k, n_experts,
                     bad);
  return hipGetLastError();
}

}  // namespace moe_fp4
