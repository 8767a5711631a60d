// Load-time re-layout of canonical expert blobs into the packed, tile-major device layout
// (see packed_layout): each (16-row tile, 128-element chunk) of a matrix becomes one
// contiguous 1 KB run of code words in the order a wavefront's lanes consume them, and
// its 64 scale bytes likewise. Rows past the matrix end are padded with zero codes and
// scale byte 127 (factor 1).
#include "moe_fp4_internal.hpp"

namespace moe_fp4 {

namespace {

// Packed word (16 bytes of codes, or one scale byte) -> (row, block) of the matrix.
__device__ __forceinline__ void tile_coords(long v, int kb, int& row, int& blk) {
  const long per_tile = 16L * kb;
  const long tile = v / per_tile;
  const long rem = v - tile * per_tile;
  const int c = (int)(rem / 64);
  const int r2 = (int)(rem - 64L * c);
  row = (int)(tile * 16 + (r2 & 15));
  blk = 4 * c + (r2 >> 4);
}

// One matrix of every expert: codes (16-byte words) when SCALES is false, scale bytes when
// true. src: canonical array of that kind for all experts (per-expert stride src_stride
// units, matrix at src_off units); dst: packed buffer (per-expert stride in bytes).
template <bool SCALES>
__global__ __launch_bounds__(256) void pack_matrix_kernel(const uint8_t* __restrict__ src, long src_stride,
                                                          long src_off, int n_experts, int rows, int tiles,
                                                          int kb, uint8_t* __restrict__ dst, size_t dst_stride,
                                                          size_t dst_off) {
  const long per_expert = (long)tiles * 16 * kb;
  const long total = per_expert * n_experts;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long)gridDim.x * blockDim.x) {
    const long e = i / per_expert;
    const long v = i - e * per_expert;
    int row, blk;
    tile_coords(v, kb, row, blk);
    const long s = e * src_stride + src_off + (long)row * kb + blk;
    uint8_t* d = dst + e * dst_stride + dst_off;
    if constexpr (SCALES) {
      d[v] = (row < rows) ? src[s] : (uint8_t)127;
    } else {
      const uint4 w = (row < rows) ? reinterpret_cast<const uint4*>(src)[s] : make_uint4(0, 0, 0, 0);
      reinterpret_cast<uint4*>(d)[v] = w;
    }
  }
}

}  // namespace

hipError_t launch_pack(const uint8_t* codes, const uint8_t* scales, int n_experts, int hidden,
                       int inter, uint8_t* packed, hipStream_t s) {
  const PackedLayout L = packed_layout(hidden, inter);
  const long hi = (long)hidden * inter;
  const long code_units = 3 * hi / 2 / 16;  // canonical per-expert strides
  const long scale_bytes = 3 * hi / kBlock;
  for (int m = 0; m < 3; ++m) {
    const MatLayout& M = L.m[m];
    const long per_expert = (long)M.tiles * 16 * M.kb;
    long blocks = (per_expert * n_experts + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipError_t e = launch_kernel(kKindPack, pack_matrix_kernel<false>, dim3((unsigned)blocks), dim3(256),
                                 0, s, codes, code_units, (long)m * (hi / 2 / 16), n_experts, M.rows,
                                 M.tiles, M.kb, packed, L.stride, M.codes);
    if (e != hipSuccess) return e;
    e = launch_kernel(kKindPack, pack_matrix_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s,
                      scales, scale_bytes, (long)m * (hi / kBlock), n_experts, M.rows, M.tiles, M.kb,
                      packed, L.stride, M.scales);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe_fp4
