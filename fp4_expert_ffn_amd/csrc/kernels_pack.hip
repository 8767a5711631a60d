// Load-time re-layout of canonical expert blobs into the packed device layout.
// The packed layout keeps each matrix row-major with its 32-code blocks contiguous (one
// 16-byte load per block, 64 blocks = 1 KB per wavefront load) and places every expert's
// codes and scales in one 256-byte-aligned region, so the compute kernels address an
// expert with a single base pointer.
#include "moe_fp4_internal.hpp"

namespace moe_fp4 {

namespace {

__global__ __launch_bounds__(256) void pack_kernel(const uint4* __restrict__ codes,
                                                   const uint4* __restrict__ scales,
                                                   long code_chunks, long scale_chunks,
                                                   long stride_chunks, int n_experts,
                                                   uint4* __restrict__ packed) {
  const long per_expert = code_chunks + scale_chunks;
  const long total = per_expert * n_experts;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long)gridDim.x * blockDim.x) {
    const long e = i / per_expert;
    const long c = i - e * per_expert;
    const uint4 v = (c < code_chunks) ? codes[e * code_chunks + c]
                                      : scales[e * scale_chunks + (c - code_chunks)];
    packed[e * stride_chunks + c] = v;
  }
}

}  // namespace

hipError_t launch_pack(const uint8_t* codes, const uint8_t* scales, int n_experts, int hidden,
                       int inter, uint8_t* packed, hipStream_t s) {
  const PackedLayout L = packed_layout(hidden, inter);
  const size_t hi = (size_t)hidden * inter;
  const long code_chunks = (long)(3 * hi / 2 / 16);
  const long scale_chunks = (long)(3 * hi / kBlock / 16);
  const long total = (code_chunks + scale_chunks) * n_experts;
  long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(codes), reinterpret_cast<const uint4*>(scales),
                     code_chunks, scale_chunks, (long)(L.stride / 16), n_experts,
                     reinterpret_cast<uint4*>(packed));
  return hipGetLastError();
}

}  // namespace moe_fp4
