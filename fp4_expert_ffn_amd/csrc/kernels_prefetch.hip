// Speculative expert prefetch ([8GB-GPU], section 提速之路：v1 到 v4, v4: the router of layer
// l + 1 applied to layer l's input predicts the next layer's experts, whose weights are then
// fetched ahead of need). Here the experts are already resident in HBM, so the only place
// to fetch them into is the memory-side cache that every HBM read passes through: this
// kernel reads the chosen matrices of the given experts with ordinary (cached) loads, so
// that a later FFN call on them reads from that cache instead of HBM. It writes nothing but
// keeps its loads alive through a data-dependent store to `sink` that practically never
// executes. Opt-in; the FFN does not depend on it.
#include <algorithm>

#include "moe_fp4_device.hpp"
#include "moe_fp4_internal.hpp"

namespace moe_fp4 {

namespace {

// Workgroups of one prefetch launch (all ranges together); overridable at build time.
#ifndef MOE_FP4_PF_WORKGROUPS
#define MOE_FP4_PF_WORKGROUPS 2048
#endif
constexpr int kPfThreads = 256;
constexpr int kPfUnroll = 4;  // 16-byte loads in flight per lane
constexpr uint32_t kPfNever = 0x7F4A7C15u;

// Byte ranges of one packed expert to read: up to the three code regions and the three
// scale regions (16-byte multiples, 256-byte aligned offsets).
struct PfRanges {
  unsigned long long off[6];
  unsigned long long len[6];
  int n;
};

// Workgroup b: id index b / (n * parts), range (b / parts) % n, part b % parts of it.
__global__ __launch_bounds__(kPfThreads) void prefetch_kernel(const int32_t* __restrict__ ids,
                                                              const uint8_t* __restrict__ packed,
                                                              size_t stride, int n_experts,
                                                              PfRanges R, int parts,
                                                              uint32_t* __restrict__ sink) {
  const long b = blockIdx.x;
  const long per_id = (long)R.n * parts;
  const int which = (int)(b / per_id);
  const int rem = (int)(b - (long)which * per_id);
  const int r = rem / parts;
  const int part = rem - r * parts;
  const int e = ids[which];
  if (e < 0 || e >= n_experts) return;  // whole workgroup
  const uint4* base = reinterpret_cast<const uint4*>(packed + (size_t)e * stride + R.off[r]);
  const size_t n16 = R.len[r] / 16;
  const size_t step = (size_t)parts * kPfThreads;
  size_t i = (size_t)part * kPfThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (size_t)(kPfUnroll - 1) * step < n16; i += (size_t)kPfUnroll * step) {
    uint4 v[kPfUnroll];
#pragma unroll
    for (int u = 0; u < kPfUnroll; ++u) v[u] = base[i + (size_t)u * step];
#pragma unroll
    for (int u = 0; u < kPfUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += step) {
    const uint4 v = base[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == kPfNever) *sink = acc;
}

}  // namespace

hipError_t launch_prefetch_experts(const int32_t* ids, int n_ids, const uint8_t* packed,
                                   int n_experts, int hidden, int inter, int matrices,
                                   uint32_t* sink, hipStream_t s) {
  const PackedLayout L = packed_layout(hidden, inter);
  PfRanges R{};
  for (int m = 0; m < 3; ++m) {
    if (!(matrices & (1 << m))) continue;
    const size_t words = (size_t)L.m[m].tiles * 16 * L.m[m].kb;  // 16-byte code words
    R.off[R.n] = L.m[m].codes;
    R.len[R.n] = words * 16;
    ++R.n;
    R.off[R.n] = L.m[m].scales;
    R.len[R.n] = (words + 15) / 16 * 16;  // scale bytes, read in 16-byte words
    ++R.n;
  }
  // about MOE_FP4_PF_WORKGROUPS workgroups in all, at least one per range
  const int parts = std::max(1, std::min(256, MOE_FP4_PF_WORKGROUPS / std::max(1, n_ids * R.n)));
  const long blocks = (long)n_ids * R.n * parts;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  return launch_kernel(kKindPrefetch, prefetch_kernel, dim3((unsigned)blocks), dim3(kPfThreads),
                       0, s, ids, packed, L.stride, n_experts, R, parts, sink);
}

}  // namespace moe_fp4
