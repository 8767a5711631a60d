// Router: logits = W_r x in fp64, then top-k selection and softmax over the selection.
// Ids never leave the device ([8GB-GPU], section 提速之路：v1 到 v4: one host round trip per
// expert on the indices was a measured cost; here there is none).
#include <math.h>

#include <algorithm>

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
  constexpr int kBatch = 8;  // 16-byte loads of x and W_r in flight per lane
  for (int c0 = lane; c0 < chunks; c0 += 64 * kBatch) {
    uint4 a[kBatch], b[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = c0 + u * 64;
      a[u] = (c < chunks) ? xv[c] : make_uint4(0, 0, 0, 0);
      b[u] = (c < chunks) ? wv[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const uint32_t av[4] = {a[u].x, a[u].y, a[u].z, a[u].w};
      const uint32_t bv[4] = {b[u].x, b[u].y, b[u].z, b[u].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float p0 = bf16_bits_to_f32(av[q] & 0xffffu) * bf16_bits_to_f32(bv[q] & 0xffffu);
        const float p1 = bf16_bits_to_f32(av[q] >> 16) * bf16_bits_to_f32(bv[q] >> 16);
        acc += (double)p0;
        acc += (double)p1;
      }
    }
  }
  acc = wave_sum_f64(acc);
  if (lane == 0) logits[(size_t)t * E + e] = acc;
}

// One wave per token: top-k selection and softmax weights (see wave_topk).
template <typename V, int kPer>
__global__ __launch_bounds__(kThreads) void topk_kernel(const V* __restrict__ logits, int T, int E,
                                                        int k, int32_t* __restrict__ ids,
                                                        float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const long t = (long)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  int sid[8];
  float sw[8];
  wave_topk<kPer>(logits + (size_t)t * E, E, k, lane, sid, sw);
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        ids[(size_t)t * k + j] = sid[j];
        w[(size_t)t * k + j] = sw[j];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Batch-1 routing in one launch. Workgroup g computes the logits of kRouteRowsPerWG
// consecutive experts (kRouteKSplit wavefronts per row group, each over its part of K) and
// publishes each as a self-checking record: its fp64 bits and those bits XOR a key derived
// from the call's epoch. Workgroup 0 polls the records themselves with agent-coherent
// loads until every check word matches its value, so the logits arrive with the
// readiness test (no flag round trip, then no reload), and selects the top-k. A record
// read half old and half new fails the check, as does one left by an earlier call.
// The epoch is not reset: every workgroup reads the epoch word at start, and workgroup 0
// stores epoch + 1 as the next call's epoch once it has seen every record (so every
// workgroup has read it). No atomic read-modify-write is needed (contended atomics across
// the eight XCDs cost tens of microseconds at this width), and the initial contents of the
// synchronisation words do not matter. The wait is bounded, so the kernel always ends: when
// a record is still missing after spin_limit polls, workgroup 0 gives up, writes ids -1 and
// weights 0 (ids that every FFN path skips and moe_fp4_validate_ids counts) and stores a
// failure mark in the synchronisation area. A workgroup that starts after the give-up may
// publish this call's logits under a key a later call would accept, so the mark is sticky:
// every later call on the area writes ids -1 as well, until the area is cleared
// (moe_fp4_route_reset), and moe_fp4_route_status reports it.
// ---------------------------------------------------------------------------------------
// Launch shape, measured on MI355X (H 4096, 384 experts): more workgroups with fewer bytes
// each shorten the GEMV; overridable at build time.
#ifndef MOE_FP4_ROUTE_ROWS_PER_WAVE
#define MOE_FP4_ROUTE_ROWS_PER_WAVE 1  // router rows of one wavefront
#endif
#ifndef MOE_FP4_ROUTE_WAVES
#define MOE_FP4_ROUTE_WAVES 8          // wavefronts per workgroup (at least 4: the norm helpers)
#endif
#ifndef MOE_FP4_ROUTE_KSPLIT
#define MOE_FP4_ROUTE_KSPLIT 4         // wavefronts sharing the K range of one row group
#endif
constexpr int kRouteRowsPerWave = MOE_FP4_ROUTE_ROWS_PER_WAVE;
constexpr int kRouteWaves = MOE_FP4_ROUTE_WAVES;
constexpr int kRouteKSplit = MOE_FP4_ROUTE_KSPLIT;
constexpr int kRouteRowsPerWG = kRouteRowsPerWave * kRouteWaves / kRouteKSplit;
constexpr int kRouteThreads = kRouteWaves * 64;
static_assert(kRouteWaves >= 4 && kRouteWaves % kRouteKSplit == 0 && kRouteRowsPerWG <= 64,
              "route launch shape");
constexpr unsigned kSpinLimit = 1u << 22;
constexpr int kRouteRecOffset = 16;  // sync words before the logit records (64 bytes)
constexpr int kRouteMarkWord = 2;    // 64-bit failure mark at sync words 2..3
constexpr uint64_t kRouteFailMark = 0x4D4F4546344E4F47ull;  // a failed wait ("MOEF4NOG")

// Epoch -> record key (the splitmix64 finaliser: consecutive epochs give unrelated keys).
__device__ __forceinline__ uint64_t route_record_key(uint32_t epoch) {
  uint64_t z = (uint64_t)epoch + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

typedef unsigned route_u32x4 __attribute__((ext_vector_type(4)));

// One 16-byte record read at the agent-coherent level (the form of an agent-scope atomic
// load), waited for at once.
__device__ __forceinline__ route_u32x4 ld_record(const uint64_t* p) {
  route_u32x4 v;
  __asm__ volatile("global_load_dwordx4 %0, %1, off sc1\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
  return v;
}

// NIT > 0: the router input is computed here from a residual stream: r_out = r_in + y_prev
// and x = bf16(r_out / rms) (the shared row helpers, so the bits equal the standalone norm
// kernel's). Every workgroup normalises the row into LDS for its own GEMV (waves 0-3, the
// helpers' 256 threads) and writes its 1/G slice of r_out and x_out for the later kernels.
template <int PER, int NIT>
__global__ __launch_bounds__(kRouteThreads) void route_decode_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int H, int E, int k,
    uint32_t* __restrict__ sync, int32_t* __restrict__ ids,
    float* __restrict__ w, const float* __restrict__ r_in, const uint16_t* __restrict__ y_prev,
    float* __restrict__ r_out, uint16_t* __restrict__ x_out, float eps, unsigned spin_limit) {
  const int G = gridDim.x;
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const uint32_t target = sync[0] + 1u;
  const uint64_t key = route_record_key(target);
  uint64_t* rec = reinterpret_cast<uint64_t*>(sync + kRouteRecOffset);

  extern __shared__ uint4 s_x[];  // NIT > 0: the normalised row, H / 8 words
  if constexpr (NIT > 0) {
    __shared__ double npart[kNormRowThreads / 64];
    float4 ra[NIT], rb[NIT];
    if (tid < kNormRowThreads) {  // wave-uniform
      double ss = norm_row_add<NIT>(r_in, y_prev, H, tid, ra, rb);
      ss = wave_sum_f64(ss);
      if (lane == 0) npart[wv] = ss;
    }
    __syncthreads();
    if (tid < kNormRowThreads) {
      const double inv = norm_row_inv(npart, H, eps);
      const int n8 = H / 8;
      const int s0 = (int)((long)g * n8 / G), s1 = (int)((long)(g + 1) * n8 / G);
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int q = tid + it * kNormRowThreads;  // group of 8 elements
        if (q < n8) {
          const uint4 xo = norm_row_pack8(ra[it], rb[it], inv);
          s_x[q] = xo;
          if (q >= s0 && q < s1) {
            *reinterpret_cast<uint4*>(x_out + 8 * q) = xo;
            *reinterpret_cast<float4*>(r_out + 8 * q) = ra[it];
            *reinterpret_cast<float4*>(r_out + 8 * q + 4) = rb[it];
          }
        }
      }
    }
    __syncthreads();
  }

  // GEMV, fp64 accumulation of the exact bf16 x bf16 products (same order for every row).
  // Wave wv takes rows row0 .. row0 + kRouteRowsPerWave - 1 over its part ks of the K range.
  const int ks = wv % kRouteKSplit;
  const int row0 = g * kRouteRowsPerWG + (wv / kRouteKSplit) * kRouteRowsPerWave;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const int chunks = H / 8;
  const int c_beg = ks * chunks / kRouteKSplit, c_end = (ks + 1) * chunks / kRouteKSplit;
  double acc[kRouteRowsPerWave];
#pragma unroll
  for (int r = 0; r < kRouteRowsPerWave; ++r) acc[r] = 0.0;
  constexpr int kBatch = 8 / kRouteKSplit > 0 ? 8 / kRouteKSplit : 1;
  for (int c0 = c_beg + lane; c0 < c_end; c0 += 64 * kBatch) {
    uint4 a[kBatch], b[kRouteRowsPerWave][kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = c0 + u * 64;
      if constexpr (NIT > 0)
        a[u] = (c < c_end) ? s_x[c] : make_uint4(0, 0, 0, 0);
      else
        a[u] = (c < c_end) ? xv[c] : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < kRouteRowsPerWave; ++r) {
        const int row = min(row0 + r, E - 1);
        b[r][u] = (c < c_end) ? reinterpret_cast<const uint4*>(wr + (size_t)row * H)[c]
                              : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const uint32_t av[4] = {a[u].x, a[u].y, a[u].z, a[u].w};
#pragma unroll
      for (int r = 0; r < kRouteRowsPerWave; ++r) {
        const uint32_t bv[4] = {b[r][u].x, b[r][u].y, b[r][u].z, b[r][u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float p0 = bf16_bits_to_f32(av[q] & 0xffffu) * bf16_bits_to_f32(bv[q] & 0xffffu);
          const float p1 = bf16_bits_to_f32(av[q] >> 16) * bf16_bits_to_f32(bv[q] >> 16);
          acc[r] += (double)p0;
          acc[r] += (double)p1;
        }
      }
    }
  }
  // The workgroup's logits go through LDS to wave 0, which writes each one's record with
  // relaxed agent-scope atomic stores (written through to the agent-coherent level, so no
  // L2 write-back fence is needed). The K parts of a row are added in ascending part order.
  __shared__ double s_part[kRouteWaves * kRouteRowsPerWave];
#pragma unroll
  for (int r = 0; r < kRouteRowsPerWave; ++r) {
    acc[r] = wave_sum_f64(acc[r]);
    if (lane == 0) s_part[wv * kRouteRowsPerWave + r] = acc[r];
  }
  __syncthreads();
  if (wv == 0) {
    const int row = g * kRouteRowsPerWG + lane;
    if (lane < kRouteRowsPerWG && row < E) {
      const int rg = lane / kRouteRowsPerWave, r = lane - rg * kRouteRowsPerWave;
      double logit = s_part[rg * kRouteKSplit * kRouteRowsPerWave + r];
#pragma unroll
      for (int p = 1; p < kRouteKSplit; ++p)
        logit += s_part[(rg * kRouteKSplit + p) * kRouteRowsPerWave + r];
      const uint64_t vb = (uint64_t)__double_as_longlong(logit);
      __hip_atomic_store(&rec[2 * row], vb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&rec[2 * row + 1], vb ^ key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (g != 0) return;

  // workgroup 0: the failure mark of an earlier call, then every record, checked, into LDS
  // for the selection (at most spin_limit polls per record)
  uint64_t* mark = reinterpret_cast<uint64_t*>(sync + kRouteMarkWord);
  const bool failed_before =
      __hip_atomic_load(mark, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == kRouteFailMark;
  __shared__ double s_lg[64 * PER];
  __shared__ int s_missing;
  if (tid == 0) s_missing = 0;
  __syncthreads();
  bool missing = false;
  for (int f = tid; f < E; f += kRouteThreads) {
    unsigned n = 0;
    uint64_t vb = 0;
    bool ok = false;
    while (!failed_before && n < spin_limit) {
      const route_u32x4 r = ld_record(&rec[2 * f]);
      vb = ((uint64_t)r.y << 32) | r.x;
      const uint64_t ck = ((uint64_t)r.w << 32) | r.z;
      if (ck == (vb ^ key)) {
        ok = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      ++n;
    }
    missing |= !ok;
    s_lg[f] = __longlong_as_double((long long)vb);
  }
  if (missing) s_missing = 1;  // any thread; a plain store of the same value
  __syncthreads();
  const bool fail = failed_before || s_missing != 0;  // workgroup-uniform
  if (wv == 0) {
    if (!fail) {
      int sid[8];
      float sw[8];
      wave_topk<PER>(s_lg, E, k, lane, sid, sw);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < k && lane == j) {
          ids[j] = sid[j];
          w[j] = sw[j];
        }
      }
      if (lane == 0) sync[0] = target;
    } else {
      if (lane < k) {
        ids[lane] = -1;
        w[lane] = 0.f;
      }
      if (lane == 0) __hip_atomic_store(mark, kRouteFailMark, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// moe_fp4_route_status: 1 if the synchronisation area holds the failure mark, else 0.
__global__ void route_status_kernel(const uint32_t* __restrict__ sync, int32_t* __restrict__ status) {
  if (threadIdx.x == 0) {
    const uint64_t m = __hip_atomic_load(reinterpret_cast<const uint64_t*>(sync + kRouteMarkWord),
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *status = m == kRouteFailMark ? 1 : 0;
  }
}

// moe_fp4_route_reset: zero the synchronisation area (a fill kernel, so the call can be
// captured in a graph).
__global__ __launch_bounds__(256) void route_reset_kernel(uint4* __restrict__ sync, int n16) {
  for (int i = threadIdx.x; i < n16; i += 256) sync[i] = make_uint4(0, 0, 0, 0);
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
  return launch_kernel(kKindRouterGemv, router_gemv_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       s, x, wr, T, hidden, n_experts, logits);
}

template <typename V>
hipError_t launch_topk(const V* logits, int T, int n_experts, int k, int32_t* ids, float* w,
                       hipStream_t s) {
  const dim3 grid((unsigned)(((long)T + kWaves - 1) / kWaves)), block(kThreads);
  const int per = (n_experts + 63) / 64;
  if (per <= 1) return launch_kernel(kKindTopk, topk_kernel<V, 1>, grid, block, 0, s, logits, T, n_experts, k, ids, w);
  if (per <= 2) return launch_kernel(kKindTopk, topk_kernel<V, 2>, grid, block, 0, s, logits, T, n_experts, k, ids, w);
  if (per <= 4) return launch_kernel(kKindTopk, topk_kernel<V, 4>, grid, block, 0, s, logits, T, n_experts, k, ids, w);
  if (per <= 8) return launch_kernel(kKindTopk, topk_kernel<V, 8>, grid, block, 0, s, logits, T, n_experts, k, ids, w);
  if (per <= 16) return launch_kernel(kKindTopk, topk_kernel<V, 16>, grid, block, 0, s, logits, T, n_experts, k, ids, w);
  return launch_kernel(kKindTopk, topk_kernel<V, 32>, grid, block, 0, s, logits, T, n_experts, k, ids, w);
}

template <int NIT>
hipError_t route_decode_launch(const uint16_t* x, const uint16_t* wr, int hidden, int n_experts,
                               int k, uint32_t* sync, double* logits, int32_t* ids, float* w,
                               const float* r_in, const uint16_t* y_prev, float* r_out,
                               uint16_t* x_out, float eps, hipStream_t s) {
  (void)logits;  // the batch-1 kernel keeps its logits in the records of the sync area
  const dim3 grid((unsigned)((n_experts + kRouteRowsPerWG - 1) / kRouteRowsPerWG)), block(kRouteThreads);
  const uint32_t lds = NIT > 0 ? (uint32_t)hidden * 2u : 0u;
  const int per = (n_experts + 63) / 64;
#define MOE_FP4_ROUTE_LAUNCH(P)                                                                   \
  return launch_kernel(kKindRouteDecode, route_decode_kernel<P, NIT>, grid, block, lds, s, x, wr,  \
                       hidden, n_experts, k, sync, ids, w, r_in, y_prev, r_out, x_out, eps,      \
                       route_spin_limit())
  if (per <= 2) MOE_FP4_ROUTE_LAUNCH(2);
  if (per <= 4) MOE_FP4_ROUTE_LAUNCH(4);
  if (per <= 6) MOE_FP4_ROUTE_LAUNCH(6);
  if (per <= 8) MOE_FP4_ROUTE_LAUNCH(8);
  if (per <= 16) MOE_FP4_ROUTE_LAUNCH(16);
  MOE_FP4_ROUTE_LAUNCH(32);
#undef MOE_FP4_ROUTE_LAUNCH
}

hipError_t launch_route_decode(const uint16_t* x, const uint16_t* wr, int hidden, int n_experts,
                               int k, uint32_t* sync, double* logits, int32_t* ids, float* w,
                               hipStream_t s) {
  return route_decode_launch<0>(x, wr, hidden, n_experts, k, sync, logits, ids, w, nullptr,
                                nullptr, nullptr, nullptr, 0.f, s);
}

hipError_t launch_route_decode_norm(const float* r_in, const uint16_t* y_prev, float* r_out,
                                    uint16_t* x_out, float eps, const uint16_t* wr, int hidden,
                                    int n_experts, int k, uint32_t* sync, double* logits,
                                    int32_t* ids, float* w, hipStream_t s) {
  if (hidden % 8 != 0 || hidden > 8 * 8 * kNormRowThreads) return hipErrorInvalidValue;
  const int nit = (hidden + 8 * kNormRowThreads - 1) / (8 * kNormRowThreads);
#define MOE_FP4_RN(N)                                                                            \
  return route_decode_launch<N>(nullptr, wr, hidden, n_experts, k, sync, logits, ids, w, r_in,   \
                                y_prev, r_out, x_out, eps, s)
  if (nit <= 1) MOE_FP4_RN(1);
  if (nit <= 2) MOE_FP4_RN(2);
  if (nit <= 4) MOE_FP4_RN(4);
  MOE_FP4_RN(8);
#undef MOE_FP4_RN
}

namespace {
unsigned g_route_spin_limit = kSpinLimit;
}

unsigned route_spin_limit() { return g_route_spin_limit; }

void set_route_spin_limit(long long polls) {
  g_route_spin_limit = polls < 0 ? kSpinLimit : (unsigned)std::min<long long>(polls, kSpinLimit);
}

hipError_t launch_route_status(const uint32_t* sync, int32_t* status, hipStream_t s) {
  route_status_kernel<<<dim3(1), dim3(64), 0, s>>>(sync, status);
  return hipGetLastError();
}

hipError_t launch_route_reset(uint32_t* sync, size_t bytes, hipStream_t s) {
  route_reset_kernel<<<dim3(1), dim3(256), 0, s>>>(reinterpret_cast<uint4*>(sync), (int)(bytes / 16));
  return hipGetLastError();
}

int route_decode_sync_words(int n_experts) {
  return kRouteRecOffset + 4 * n_experts;  // the epoch word, then a 16-byte record per expert
}

hipError_t launch_topk_f64(const double* logits, int T, int n_experts, int k, int32_t* ids,
                           float* w, hipStream_t s) {
  return launch_topk<double>(logits, T, n_experts, k, ids, w, s);
}

hipError_t launch_topk_f32(const float* logits, int T, int n_experts, int k, int32_t* ids,
                           float* w, hipStream_t s) {
  return launch_topk<float>(logits, T, n_experts, k, ids, w, s);
}

hipError_t launch_validate_ids(const int32_t* ids, int T, int k, int n_experts, int32_t* bad,
                               hipStream_t s) {
  validate_ids_kernel<<<dim3(1), dim3(1024), 0, s>>>(ids, (long)T * k, n_experts, bad);
  return hipGetLastError();
}

}  // namespace moe_fp4
