// Dense FP8 weights: the shared expert and the dense projections. The weights stay FP8 E4M3
// in memory and become bf16 matrix-core operands in registers ([A100-FP4], Chinese
// translation, section A100 也没有 FP8: FP8 as a storage format, converted on the way from
// memory to the matrix unit, never expanded in memory). Each [N x K] matrix carries one
// fp32 multiplier per 128 x 128 block.
//
// Packed layout (moe_fp4_fp8_pack): 16-row tiles, 128-element chunks along K. For each
// (tile, chunk) 2 KB of codes in [half h][block g][row j] order of 16-byte words, word
// (h, g, j) = codes[16 tile + j][128 chunk + 32 g + 16 h .. + 15]: a wavefront load of 1 KB
// (h fixed, lane = 16 g + j) gives every lane half of one 32-element block. Rows past N and
// blocks past K are zero codes. Then one fp32 per (tile, chunk): the multiplier of the
// 128 x 128 block holding that tile and chunk (a 16-row tile lies inside one 128-row block).
//
// GEMV kernel: a workgroup of 16 wavefronts owns 16 weight rows for up to MR tokens, whose
// rows are matrix-core rows (x staged in LDS); the waves split the K chunks. With one matrix
// the 16 rows are one tile. With two (gate and up) they are 8 rows of each: half h of a
// tile, gate rows in MFMA columns 0-7 and the same up rows in columns 8-15. The launch then
// has twice as many workgroups, enough to cover the compute units at the shared expert's
// size, and SiLU(gate) * up pairs column c with c + 8. A chunk's four MFMAs accumulate into a fresh register set that
// is then added into the running sum times the chunk's multiplier (the conversion to bf16
// is exact, so every product is exact and only fp32 sums round).
#include <algorithm>

#include "moe_fp4_device.hpp"
#include "moe_fp4_gemv.hpp"
#include "moe_fp4_internal.hpp"

namespace moe_fp4 {

namespace {

// Launch shape, overridable at build time.
#ifndef MOE_FP4_F8_WAVES
#define MOE_FP4_F8_WAVES 16   // wavefronts per workgroup (they split K)
#endif
#ifndef MOE_FP4_F8_BATCH
#define MOE_FP4_F8_BATCH 2    // chunks loaded per wave before use
#endif
constexpr int kF8Waves = MOE_FP4_F8_WAVES;
constexpr int kF8Threads = kF8Waves * 64;
constexpr int kF8Batch = MOE_FP4_F8_BATCH;
constexpr int kF8LdsBytes = 32768;      // staged activation rows per workgroup
constexpr int kF8Stage = kF8LdsBytes / (16 * kF8Threads);  // 16-byte words per thread: 2

struct Fp8Layout {
  int tiles, nch, kb;
  size_t codes_bytes, scales_off, bytes;
};

Fp8Layout fp8_layout(int rows, int cols) {
  Fp8Layout L;
  L.tiles = (rows + 15) / 16;
  L.nch = (cols + 127) / 128;
  L.kb = cols / kBlock;
  L.codes_bytes = (size_t)L.tiles * L.nch * 2048;
  L.scales_off = align_up256(L.codes_bytes);
  L.bytes = L.scales_off + align_up256((size_t)L.tiles * L.nch * 4);
  return L;
}

// one thread per 16-byte packed word, then per (tile, chunk) multiplier
__global__ __launch_bounds__(256) void fp8_pack_kernel(const uint8_t* __restrict__ codes,
                                                       const float* __restrict__ scale_inv, int N,
                                                       int K, int tiles, int nch,
                                                       uint8_t* __restrict__ packed,
                                                       size_t scales_off) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const long words = (long)tiles * nch * 128;
  if (i < words) {
    const long tc = i / 128;
    const int r = (int)(i - tc * 128);
    const int h = r / 64, g = (r / 16) % 4, j = r % 16;
    const int t = (int)(tc / nch), c = (int)(tc - (long)t * nch);
    const int row = 16 * t + j, col = 128 * c + 32 * g + 16 * h;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < N && col < K) v = *reinterpret_cast<const uint4*>(codes + (size_t)row * K + col);
    reinterpret_cast<uint4*>(packed)[i] = v;
  }
  if (i < (long)tiles * nch) {
    const int t = (int)(i / nch), c = (int)(i - (long)(i / nch) * nch);
    const int rb = (16 * t) / 128, ncb = (K + 127) / 128;
    reinterpret_cast<float*>(packed + scales_off)[i] = scale_inv[(size_t)rb * ncb + c];
  }
}

// Two E4M3 codes (the low or high half of w) -> two bf16, exact (scale 1).
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8_t{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Activation rows t0 .. t0 + m - 1 of x [T x K] into LDS with direct global -> LDS loads
// (lane L of a wave writes 16 bytes at the wave's LDS base + 16 L). Word w of row r sits at
// r * nw + (w ^ (r & 3)): rows read at one offset meet different banks.
__device__ __forceinline__ void fp8_stage_rows(const uint4* x, long t0, int m, int nw, int wv,
                                               int lane, uint4* smem) {
  const int total = m * nw;
#pragma unroll
  for (int u = 0; u < kF8Stage; ++u) {
    const int blk = (u * kF8Waves + wv) * 64;
    const int p = blk + lane;
    if (p < total) {
      const int r = p / nw, ws = p - r * nw;
      __builtin_amdgcn_global_load_lds(x + (size_t)(t0 + r) * nw + (ws ^ (r & 3)), smem + blk, 16, 0, 0);
    }
  }
}

// NMAT 2: h = bf16(silu(W0 x) * (W1 x)) [T x N]; NMAT 1: y = bf16(W0 x) [T x N].
template <int NMAT, int MR>
__global__ __launch_bounds__(kF8Threads) void fp8_gemv_kernel(const uint16_t* __restrict__ x, int T,
                                                             int K, int N, const uint8_t* p0,
                                                             const uint8_t* p1, size_t scales_off,
                                                             int tiles, int nch,
                                                             uint16_t* __restrict__ out) {
  extern __shared__ uint4 smem[];
  constexpr int kUnits = NMAT == 2 ? 2 : 1;  // workgroups per 16-row tile
  const int grp = blockIdx.x / (tiles * kUnits);
  const int unit = blockIdx.x - grp * tiles * kUnits;
  const int tile = unit / kUnits;
  const int half = unit - tile * kUnits;
  const long t0 = (long)grp * MR;
  const int m = (int)min((long)MR, (long)T - t0);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int KB = K / kBlock;
  const int nx = K / 8;

  // 1. the tokens' rows into LDS
  fp8_stage_rows(reinterpret_cast<const uint4*>(x), t0, m, nx, wv, lane, smem);

  // 2. this wave's chunks and its first batch of weights (every load issued, clamped)
  const int c_begin = wv * nch / kF8Waves;
  const int c_end = (wv + 1) * nch / kF8Waves;
  // this lane's matrix (column j: gate for j < 8, up for j >= 8 with two matrices) and its
  // word (g, row) inside each 1 KB half of a (tile, chunk)
  const bool second = NMAT == 2 && j >= 8;
  const int wrow = NMAT == 2 ? 8 * half + (j & 7) : j;
  const uint4* wl = reinterpret_cast<const uint4*>(second ? p1 : p0) + (size_t)tile * nch * 128 +
                    16 * g + wrow;
  const float* sl = reinterpret_cast<const float*>((second ? p1 : p0) + scales_off) + (size_t)tile * nch;
  uint4 a0[kF8Batch], b0[kF8Batch];
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int q = 0; q < kF8Batch; ++q) {
      const int c = max(min(c0 + q, c_end - 1), 0);
      a0[q] = ld_stream(wl + (size_t)c * 128);
      b0[q] = ld_stream(wl + (size_t)c * 128 + 64);
    }
  };
  load_batch(c_begin);
  __syncthreads();

  // A operand: row rj = min(j, m - 1) (rows >= m are never stored), words 16 c + 4 g + ms;
  // a K-tail lane (block 4 c + g past K, zero codes) reads its row's first words instead
  const char* lds = reinterpret_cast<const char*>(smem);
  const int rj = min(j, m - 1);
  uint32_t a_off[4];
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) a_off[ms] = (uint32_t)(rj * nx + 4 * g + (ms ^ (rj & 3))) * 16u;
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f};
  auto chunk = [&](int c, const uint4& lo, const uint4& hi, float sc, f32x4_t& acc) {
    const uint32_t cb = (4 * c + g < KB) ? (uint32_t)c * 256u : 0u - 64u * (uint32_t)g;
    const uint32_t wd[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    f32x4_t part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
      const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(lds + a_off[ms] + cb));
      part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, fp8x8_to_bf16(wd[2 * ms], wd[2 * ms + 1]), part,
                                                     0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = fmaf(sc, part[q], acc[q]);
  };
  for (int c0 = c_begin; c0 < c_end; c0 += kF8Batch) {
#pragma unroll
    for (int q = 0; q < kF8Batch; ++q) {
      const int c = c0 + q;
      if (c < c_end) {  // wave-uniform
        chunk(c, a0[q], b0[q], sl[c], acc0);
      }
    }
    if (c0 + kF8Batch < c_end) load_batch(c0 + kF8Batch);
  }

  // 3. partial sums over the staged rows' LDS: [wave][row][column]
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 4 * g + q;  // accumulator element q: row 4 (lane / 16) + q, column lane % 16
    if (r < m) red[(wv * MR + r) * 16 + j] = acc0[q];
  }
  __syncthreads();
  constexpr int kCols = 16 / kUnits;  // outputs per token: 16 rows, or 8 (gate, up) pairs
  if (tid < MR * kCols) {
    const int r = tid / kCols, c = tid % kCols;
    const int n = 16 * tile + kCols * half + c;
    if (r < m && n < N) {
      float v0 = 0.f, v1 = 0.f;
#pragma unroll
      for (int w = 0; w < kF8Waves; ++w) {
        v0 += red[(w * MR + r) * 16 + c];
        if constexpr (NMAT == 2) v1 += red[(w * MR + r) * 16 + c + 8];
      }
      const float v = NMAT == 2 ? silu_f32(v0) * v1 : v0;
      out[(size_t)(t0 + r) * N + n] = f32_to_bf16_rne(v);
    }
  }
}

// Tokens per workgroup: the largest power of two <= min(T, 4) whose bf16 rows fit in
// kF8LdsBytes.
int fp8_rows(int T, int K) {
  int mr = 4;
  while (mr > 1 && (mr > T || (size_t)mr * K * 2 > (size_t)kF8LdsBytes)) mr /= 2;
  return mr;
}

template <int NMAT, int MR>
hipError_t fp8_gemv_launch(const uint16_t* x, int T, int K, int N, const uint8_t* p0,
                           const uint8_t* p1, uint16_t* out, hipStream_t s) {
  const Fp8Layout L = fp8_layout(N, K);
  const long groups = (T + MR - 1) / MR;
  const long grid = groups * L.tiles * NMAT;  // two matrices: a workgroup per half tile
  if (grid > 0x7fffffffL) return hipErrorInvalidValue;
  const uint32_t lds = (uint32_t)std::max(MR * (K / 8) * 16, kF8Waves * MR * 16 * 4);
  return launch_kernel(kKindFp8Gemv, fp8_gemv_kernel<NMAT, MR>, dim3((unsigned)grid),
                       dim3(kF8Threads), lds, s, x, T, K, N, p0, p1, L.scales_off, L.tiles, L.nch,
                       out);
}

template <int NMAT>
hipError_t fp8_gemv(const uint16_t* x, int T, int K, int N, const uint8_t* p0, const uint8_t* p1,
                    uint16_t* out, hipStream_t s) {
  switch (fp8_rows(T, K)) {
    case 4: return fp8_gemv_launch<NMAT, 4>(x, T, K, N, p0, p1, out, s);
    case 2: return fp8_gemv_launch<NMAT, 2>(x, T, K, N, p0, p1, out, s);
    default: return fp8_gemv_launch<NMAT, 1>(x, T, K, N, p0, p1, out, s);
  }
}

}  // namespace

size_t fp8_packed_bytes(int rows, int cols) { return fp8_layout(rows, cols).bytes; }

hipError_t launch_fp8_pack(const uint8_t* codes, const float* scale_inv, int rows, int cols,
                           uint8_t* packed, hipStream_t s) {
  const Fp8Layout L = fp8_layout(rows, cols);
  const long words = (long)L.tiles * L.nch * 128;
  return launch_kernel(kKindPack, fp8_pack_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0,
                       s, codes, scale_inv, rows, cols, L.tiles, L.nch, packed, L.scales_off);
}

hipError_t launch_fp8_linear(const uint16_t* x, int T, const uint8_t* packed, int rows, int cols,
                             uint16_t* y, hipStream_t s) {
  return fp8_gemv<1>(x, T, cols, rows, packed, packed, y, s);
}

hipError_t launch_fp8_swiglu(const uint16_t* x, int T, const uint8_t* gate, const uint8_t* up,
                             int inter, int hidden, uint16_t* h, hipStream_t s) {
  return fp8_gemv<2>(x, T, hidden, inter, gate, up, h, s);
}

}  // namespace moe_fp4
