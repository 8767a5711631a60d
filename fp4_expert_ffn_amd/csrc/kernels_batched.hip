// Batched routed expert FFN: (token, slot) pairs grouped by expert, then a grouped GEMM on the
// block-scaled matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4). Used where several tokens
// share an expert, so each expert's FP4 weights are streamed once per 64 of its tokens
// instead of once per token.
//
// 1. sort_kernel: histogram of the valid ids over experts, exclusive scan, scatter of pair
//    indices into expert order (perm), and a table of 64-row M-blocks per expert. The order
//    of pairs inside an expert's group is not fixed (LDS atomics), and nothing depends on
//    it: every MFMA row is computed on its own, with the same K order.
// 2. quant_x_kernel: x -> two-term MXFP6 (E2M3) hi + lo with one ue8m0 scale per 32 elements
//    each (lo = the same quantisation of x - hi). One 8-bit or 6-bit term alone does not
//    meet the output tolerance; two E2M3 terms do, and E2M3 codes enter the block-scaled
//    MFMA at the FP4 rate, twice the FP8 one. The scale exponent is the smallest X with
//    max|v| <= vmax * 2^X (vmax 7.5 for E2M3, 448 for E4M3), so no element overflows the
//    element range. The opt-in single-term mode (TERMS = 1) is one E4M3 term: DeepSeek's own
//    FP8 activation numerics with ue8m0 scales ([8GB-GPU], section RTX 50xx 上的三个从不抛错的
//    Bug). Building with MOE_FP4_GROUPED_FMT=0 makes the two-term path E4M3 hi + lo instead.
// 3. gemm_gate_up_kernel: per (M-block, 128 rows of I): g and u for 128 rows of gate and up,
//    h = silu(g) * u, quantised in the epilogue to the same two terms (blocks of 32 along I).
// 4. gemm_down_kernel: per (M-block, 128 rows of H): y_e = W_down h, times the pair's router
//    weight, written fp32 per pair.
// 5. combine_kernel: y[t] = sum of the token's valid pairs in canonical slot order (ascending
//    expert id, then weight bits, then slot) -> bf16.
//
// Operand layout of the block-scaled MFMA (16 x 16 x 128), measured on gfx950:
//  * B, FP4 (4 of the 8 operand dwords used): lane 16 g + j holds column j, K = 32 g + e for
//    nibble e (low nibble first). One packed tile-major word (tile, chunk c, g, j) is exactly
//    this operand for weight rows tile * 16 .. + 15 and K = 128 c .. 128 c + 127, so a
//    wavefront reads its B operand as one contiguous 1 KB load.
//  * A, FP8 (8 dwords): lane 16 g + r holds row r; byte e sits at K = 64 (e / 16) + 16 g + e % 16,
//    i.e. two 16-byte pieces of the row at K offsets 16 g and 64 + 16 g.
//  * A, FP6 E2M3 (6 of the 8 dwords): lane 16 g + r holds row r, K = 32 g + s at bits 6 s: one
//    lane carries one whole K-block of its row, 24 bytes.
//  * Scales: lane (row or column, g) supplies the ue8m0 byte of K-block g (K = 32 g .. + 31)
//    of its row / column (operand byte 0).
//  * C: row i, column j at lane j + 16 (i / 4), element i % 4.
#include <algorithm>

#include "moe_fp4_device.hpp"
#include "moe_fp4_internal.hpp"

// B sets of the grouped gate/up K loop (1-3: how many chunks ahead its B words load) and its
// A staging depth (1, or 2 with 2 B sets: chunks between an A load and its LDS store). With
// 4 B words per wave 3 sets were 1-2 % ahead of 2 (8192 and 32768 tokens); with the 6 words
// of the default shape 3 sets spill and 2 beat 1 by 4-6 %. A depth 2 was no faster than 1
// with either shape (6.78 against 6.71 ms at 32768 tokens with six words).
#ifndef MOE_FP4_GU_BSETS
#define MOE_FP4_GU_BSETS 2
#endif
#ifndef MOE_FP4_GU_ADEPTH
#define MOE_FP4_GU_ADEPTH 1
#endif
#ifndef MOE_FP4_GU_WPE
#define MOE_FP4_GU_WPE 2  // wavefronts per SIMD the gate/up kernel is compiled for
#endif

namespace moe_fp4 {

namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Weight words are read once per M-block. Where an expert has one M-block (up to 64 of its
// tokens), non-temporal loads keep them out of the way of the reused activation rows in the
// caches; where its tokens fill several M-blocks, ordinary loads leave the tile in L2 for the
// other blocks' workgroups, which the XCD-aware order runs close in time on the same L2
// (measured at 8192 and 32768 tokens: gate/up 8-12 % and down 15-21 % faster; at 64 and
// 1024 tokens the non-temporal form is 3-6 % faster).
template <bool NT>
__device__ __forceinline__ uint4 ld_w16(const uint8_t* p) {
  if constexpr (NT) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}

constexpr int kBWaves = 4;
constexpr int kBThreads = kBWaves * 64;
// Gate/up: 16-row tiles per wave and matrix (B words per wave: twice that, at most 6). Three
// tiles (h columns per workgroup 192, so 2880 is 15 whole tiles) against two, both at 2 waves
// per SIMD: gate/up 2.43 -> 2.04 ms at 8192 tokens, 8.12 -> 6.96 ms at 32768. Each A operand
// read from LDS then feeds six B words instead of four.
#ifndef MOE_FP4_GU_NS
#define MOE_FP4_GU_NS 3
#endif
constexpr int kNS = MOE_FP4_GU_NS;
static_assert(kNS >= 1 && 2 * kNS <= 6, "gate/up B words per wave");
constexpr int kBN = 16 * kNS * kBWaves; // weight rows per workgroup
// Down: 16-row tiles of W_down per wave, its wavefronts per SIMD and B sets. Measured with the
// E2M3 operands: 4 tiles at 2 waves per SIMD with 2 B sets took down from 2.01 to 1.87 ms at
// 8192 tokens (6.29 to 6.20 at 32768) against 2 tiles at 4 waves per SIMD with one set; 5
// tiles with 2 sets from 1.63 to 1.50 ms (5.19 to 4.78); 6 tiles (384 rows of H per
// workgroup, 248 registers once the A operands needed no masks) from 1.48 to 1.38 ms (4.68
// to 4.40).
#ifndef MOE_FP4_DN_NS
#define MOE_FP4_DN_NS 6
#endif
#ifndef MOE_FP4_DN_WPE
#define MOE_FP4_DN_WPE 2
#endif
#ifndef MOE_FP4_DN_BSETS
#define MOE_FP4_DN_BSETS 2
#endif
constexpr int kDNS = MOE_FP4_DN_NS;
static_assert(kDNS >= 1 && kDNS <= 6, "down B words per wave");
constexpr int kBND = 16 * kDNS * kBWaves;  // rows of H per down workgroup
constexpr int kMSub = kBlockRows / 16;  // 16-row MFMA subtiles per M-block
constexpr int kSortThreads = 1024;
constexpr int kSortMaxGroups = 256;        // workgroups of the split sort
constexpr long kSortSplitMinPairs = 8192;  // pairs from which the sort is split (measured)

// ---------------------------------------------------------------------------------------
// MXFP8 (E4M3) encoding of one 32-element block, one or two terms.
// ---------------------------------------------------------------------------------------
// Smallest X with a <= 448 * 2^X (448 = 1.75 * 2^8, the largest E4M3 value), clamped to the
// ue8m0 range; a == 0 gives -127.
__device__ __forceinline__ int mx_exponent(float a) {
  if (!(a > 0.f)) return -127;
  const uint32_t b = __float_as_uint(a);
  int E = (int)((b >> 23) & 0xff) - 127;
  uint32_t man = b & 0x7fffffu;
  if (E == -127) {  // subnormal: normalise
    const int sh = __clz((int)man) - 8;
    man = (man << sh) & 0x7fffffu;
    E = -126 - sh;
  }
  // mantissa <= 1.75  <=>  man <= 0.75 * 2^23
  int X = (man <= 0x600000u) ? E - 8 : E - 7;
  return max(-127, min(127, X));
}

// v[0..31] (fp32) -> hi, lo E4M3 bytes (16-byte words h0,h1 / l0,l1 in element order) and
// their scale bytes; TERMS = 1 encodes hi only (lo zero, scale byte 127).
template <int TERMS>
__device__ __forceinline__ void mx8_encode_block(const float (&v)[32], uint4& h0, uint4& h1,
                                                 uint4& l0, uint4& l1, uint32_t& sh,
                                                 uint32_t& sl) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int X = mx_exponent(amax);
  uint32_t hw[8];
  float r[32];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    int w = 0;
    w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * d], -X), ldexpf(v[4 * d + 1], -X), w, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * d + 2], -X), ldexpf(v[4 * d + 3], -X), w, true);
    hw[d] = (uint32_t)w;
    if constexpr (TERMS == 1) continue;
    // residual against the decoded hi value (exact in fp32)
    r[4 * d + 0] = v[4 * d + 0] - ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)hw[d], 0), X);
    r[4 * d + 1] = v[4 * d + 1] - ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)hw[d], 1), X);
    r[4 * d + 2] = v[4 * d + 2] - ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)hw[d], 2), X);
    r[4 * d + 3] = v[4 * d + 3] - ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)hw[d], 3), X);
  }
  h0 = make_uint4(hw[0], hw[1], hw[2], hw[3]);
  h1 = make_uint4(hw[4], hw[5], hw[6], hw[7]);
  sh = (uint32_t)(X + 127);
  if constexpr (TERMS == 1) {
    l0 = l1 = make_uint4(0, 0, 0, 0);
    sl = 127u;
    return;
  }
  float rmax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) rmax = fmaxf(rmax, fabsf(r[i]));
  const int Xl = mx_exponent(rmax);
  uint32_t lw[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    int w = 0;
    w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(r[4 * d], -Xl), ldexpf(r[4 * d + 1], -Xl), w, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(r[4 * d + 2], -Xl), ldexpf(r[4 * d + 3], -Xl), w, true);
    lw[d] = (uint32_t)w;
  }
  l0 = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  l1 = make_uint4(lw[4], lw[5], lw[6], lw[7]);
  sl = (uint32_t)(Xl + 127);
}

// ---------------------------------------------------------------------------------------
// MXFP6 (E2M3) encoding of one 32-element block, two terms: the default activation format
// of the two-term grouped path. E2M3 codes enter the block-scaled MFMA at the FP4 rate
// (twice the FP8 rate), and take 24 bytes per block instead of 32.
// ---------------------------------------------------------------------------------------
constexpr int kFmtE4M3 = 0;  // activation formats: the MFMA's A-format codes
constexpr int kFmtE2M3 = 2;
#ifndef MOE_FP4_GROUPED_FMT
#define MOE_FP4_GROUPED_FMT 2  // two-term grouped path: 2 = E2M3 (FP6), 0 = E4M3 (FP8)
#endif
// format of a path: TERMS = 1 is the one-term FP8 mode
template <int TERMS>
constexpr int act_fmt() { return TERMS == 2 ? MOE_FP4_GROUPED_FMT : kFmtE4M3; }
template <int F>
constexpr int fmt_blk_bytes() { return F == kFmtE2M3 ? 24 : 32; }  // bytes per block and term
// LDS row of one 128-element chunk: hi | lo | pad (E2M3: 96 | 96 | 16, E4M3: 128 | 128 | 16)
template <int F>
constexpr int fmt_pitch() { return 2 * 4 * fmt_blk_bytes<F>() + 16; }

// Smallest X with a <= 7.5 * 2^X (7.5 = 1.875 * 2^2, the largest E2M3 value), clamped to the
// ue8m0 range; a == 0 gives -127.
__device__ __forceinline__ int mx6_exponent(float a) {
  if (!(a > 0.f)) return -127;
  const uint32_t b = __float_as_uint(a);
  int E = (int)((b >> 23) & 0xff) - 127;
  uint32_t man = b & 0x7fffffu;
  if (E == -127) {  // subnormal: normalise
    const int sh = __clz((int)man) - 8;
    man = (man << sh) & 0x7fffffu;
    E = -126 - sh;
  }
  // mantissa <= 1.875  <=>  man <= 0.875 * 2^23
  const int X = (man <= 0x700000u) ? E - 2 : E - 1;
  return max(-127, min(127, X));
}

typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef unsigned v6u_t __attribute__((ext_vector_type(6)));

// v[0..31] / 2^X -> 32 E2M3 codes, code i at bits 6 i of six dwords (the order of the MFMA's
// E2M3 A operand: one lane's 32 consecutive K values), rounded to nearest with ties to the
// even code. v_cvt_scalef32_2xpk16_fp6_f32 divides by the scale operand's power of two and
// interleaves its two 16-value sources (code 2 k from the first, 2 k + 1 from the second),
// so the even and odd values go in separately. It reads its sources after writing part of
// its result, and the compiler's allocation may place the result over them (measured:
// values 12..31 then came out wrong); the asm's early-clobber result keeps them apart.
__device__ __forceinline__ v6u_t cvt_e2m3_x32(const float (&v)[32], int X) {
  v16f_t ev, od;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    ev[i] = v[2 * i];
    od[i] = v[2 * i + 1];
  }
  const float sc = __uint_as_float((uint32_t)(X + 127) << 23);  // 2^X (exponent field only)
  v6u_t r;
  __asm__("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3" : "=&v"(r) : "v"(ev), "v"(od), "v"(sc));
  return r;
}

typedef float v32f_t __attribute__((ext_vector_type(32)));

// The 32 codes of six packed dwords back to fp32, times 2^X, by the hardware conversion
// (code i -> element i, exact: every E2M3 value times 2^X with X >= -100 is a normal fp32,
// and code 32 gives -0 like the software decode below; measured against the E2M3 definition
// for every code). The scale operand is the power of two itself. As with the conversion the
// other way, the result is kept apart from the source registers (early clobber).
__device__ __forceinline__ v32f_t e2m3_decode_x32(const v6u_t& w, int X) {
  const float sc = __uint_as_float((uint32_t)(X + 127) << 23);  // 2^X, X in [-126, 127]
  v32f_t r;
  __asm__("v_cvt_scalef32_pk32_f32_fp6 %0, %1, %2" : "=&v"(r) : "v"(w), "v"(sc));
  return r;
}

// code i of six packed dwords
__device__ __forceinline__ uint32_t e2m3_code(const v6u_t& w, int i) {
  const int bit = 6 * i, d = bit >> 5, sh = bit & 31;
  uint32_t c = w[d] >> sh;
  if (sh > 26) c |= w[d + 1] << (32 - sh);
  return c & 63u;
}

// value of an E2M3 code times 2^X (exact in fp32)
__device__ __forceinline__ float e2m3_value(uint32_t c, int X) {
  const uint32_t e = (c >> 3) & 3u, m = c & 7u;
  const uint32_t mag8 = e ? (8u + m) << (e - 1) : m;  // in units of 1/8
  const float v = ldexpf((float)mag8, X - 3);
  return (c & 32u) ? -v : v;
}

// v[0..31] (fp32) -> hi, lo E2M3 codes (six dwords each) and their scale bytes: hi = the block
// quantised with its scale, lo = the residual v - hi (exact in fp32) quantised with its own.
// E2M3 has no NaN or infinity: a block holding one gets scale byte 255 (NaN) on both terms, so
// every product with it is NaN, as the element itself would have made it.
__device__ __forceinline__ void mx6_encode_block(const float (&v)[32], v6u_t& hi, v6u_t& lo,
                                                 uint32_t& sh, uint32_t& sl) {
  float amax = 0.f;
  bool finite = true;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    amax = fmaxf(amax, fabsf(v[i]));
    finite = finite && fabsf(v[i]) <= 3.4028234663852886e38f;  // false for NaN and +-inf
  }
  const int X = mx6_exponent(amax);
  hi = cvt_e2m3_x32(v, X);
  float r[32];
  float rmax = 0.f;
  if (X >= -100) {  // the residual against the hardware decode of hi
    const v32f_t hv = e2m3_decode_x32(hi, X);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      r[i] = v[i] - hv[i];
      rmax = fmaxf(rmax, fabsf(r[i]));
    }
  } else {  // tiny blocks: hi's values may be subnormal; decoded in software
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      r[i] = v[i] - e2m3_value(e2m3_code(hi, i), X);
      rmax = fmaxf(rmax, fabsf(r[i]));
    }
  }
  const int Xl = mx6_exponent(rmax);
  lo = cvt_e2m3_x32(r, Xl);
  sh = finite ? (uint32_t)(X + 127) : 255u;
  sl = finite ? (uint32_t)(Xl + 127) : 255u;
}

// ---------------------------------------------------------------------------------------
// 1. sort by expert (one workgroup)
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int block_exclusive_scan(int v, int* sbuf) {
  // sbuf: kSortThreads ints of LDS
  const int tid = threadIdx.x;
  sbuf[tid] = v;
  __syncthreads();
  for (int off = 1; off < kSortThreads; off <<= 1) {
    const int add = (tid >= off) ? sbuf[tid - off] : 0;
    __syncthreads();
    sbuf[tid] += add;
    __syncthreads();
  }
  const int inclusive = sbuf[tid];
  __syncthreads();
  return inclusive - v;
}

__global__ __launch_bounds__(kSortThreads) void sort_kernel(
    const int32_t* __restrict__ ids, int P, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ blk_expert, int32_t* __restrict__ blk_row0,
    int32_t* __restrict__ n_blocks) {
  extern __shared__ int sm[];
  int* cnt = sm;                // E
  int* cur = sm + E;            // E
  int* boff = sm + 2 * E;       // E
  int* sbuf = sm + 3 * E;       // kSortThreads
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kSortThreads) cnt[e] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += kSortThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  // each thread owns experts [tid * per, tid * per + per)
  const int per = (E + kSortThreads - 1) / kSortThreads;
  int rows = 0, blks = 0;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < E) {
      rows += cnt[e];
      blks += (cnt[e] + kBlockRows - 1) / kBlockRows;
    }
  }
  int row_base = block_exclusive_scan(rows, sbuf);
  int blk_base = block_exclusive_scan(blks, sbuf);
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < E) {
      cur[e] = row_base;
      boff[e] = blk_base;
      offsets[e] = row_base;
      const int n = cnt[e];
      const int nb = (n + kBlockRows - 1) / kBlockRows;
      for (int b = 0; b < nb; ++b) {
        blk_expert[blk_base + b] = e;
        blk_row0[blk_base + b] = row_base + b * kBlockRows;
      }
      row_base += n;
      blk_base += nb;
    }
  }
  if (tid == kSortThreads - 1) {
    offsets[E] = row_base;
    n_blocks[0] = blk_base;
  }
  __syncthreads();
  for (int p = tid; p < P; p += kSortThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E) perm[atomicAdd(&cur[e], 1)] = p;
  }
}

// The same sort over many workgroups, for large batches (the one-workgroup sort reads every
// id and writes every perm entry from one compute unit: 175 us at 196,608 pairs). Three
// launches: each of G workgroups histograms a contiguous range of `chunk` pairs into
// cnt[g][E]; one workgroup sums the histograms per expert, scans, writes the offsets and the
// block table (as sort_kernel) and turns cnt[g][e] into workgroup g's first sorted row for
// expert e; each workgroup then scatters its range through LDS cursors starting there.
constexpr int kSortWGThreads = 256;

__global__ __launch_bounds__(kSortWGThreads) void sort_count_kernel(const int32_t* __restrict__ ids,
                                                                    int P, int E, int chunk,
                                                                    int32_t* __restrict__ cnt) {
  extern __shared__ int hist[];  // E
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kSortWGThreads) hist[e] = 0;
  __syncthreads();
  const long p0 = (long)blockIdx.x * chunk;
  const long p1 = min((long)P, p0 + chunk);
  for (long p = p0 + tid; p < p1; p += kSortWGThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kSortWGThreads) cnt[(size_t)blockIdx.x * E + e] = hist[e];
}

__global__ __launch_bounds__(kSortThreads) void sort_scan_kernel(
    int G, int E, int32_t* __restrict__ cnt, int32_t* __restrict__ offsets,
    int32_t* __restrict__ blk_expert, int32_t* __restrict__ blk_row0,
    int32_t* __restrict__ n_blocks) {
  extern __shared__ int sm[];
  int* tot = sm;              // E
  int* sbuf = sm + E;         // kSortThreads
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kSortThreads) {
    int t = 0;
    for (int g = 0; g < G; ++g) t += cnt[(size_t)g * E + e];
    tot[e] = t;
  }
  __syncthreads();
  const int per = (E + kSortThreads - 1) / kSortThreads;
  int rows = 0, blks = 0;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < E) {
      rows += tot[e];
      blks += (tot[e] + kBlockRows - 1) / kBlockRows;
    }
  }
  int row_base = block_exclusive_scan(rows, sbuf);
  int blk_base = block_exclusive_scan(blks, sbuf);
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < E) {
      offsets[e] = row_base;
      const int n = tot[e];
      const int nb = (n + kBlockRows - 1) / kBlockRows;
      for (int b = 0; b < nb; ++b) {
        blk_expert[blk_base + b] = e;
        blk_row0[blk_base + b] = row_base + b * kBlockRows;
      }
      // workgroup g's first row for expert e: after the rows of the workgroups before it
      int start = row_base;
      for (int g = 0; g < G; ++g) {
        const int c = cnt[(size_t)g * E + e];
        cnt[(size_t)g * E + e] = start;
        start += c;
      }
      row_base += n;
      blk_base += nb;
    }
  }
  if (tid == kSortThreads - 1) {
    offsets[E] = row_base;
    n_blocks[0] = blk_base;
  }
}

__global__ __launch_bounds__(kSortWGThreads) void sort_scatter_kernel(const int32_t* __restrict__ ids,
                                                                      int P, int E, int chunk,
                                                                      const int32_t* __restrict__ start,
                                                                      int32_t* __restrict__ perm) {
  extern __shared__ int cur[];  // E
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kSortWGThreads) cur[e] = start[(size_t)blockIdx.x * E + e];
  __syncthreads();
  const long p0 = (long)blockIdx.x * chunk;
  const long p1 = min((long)P, p0 + chunk);
  for (long p = p0 + tid; p < p1; p += kSortWGThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E) perm[atomicAdd(&cur[e], 1)] = (int32_t)p;
  }
}

// ---------------------------------------------------------------------------------------
// 2. x -> MX hi / lo (E2M3 two terms; E4M3 hi only for TERMS = 1), one thread per (token,
//    32-block); blocks past H are zero (scale byte 127)
// ---------------------------------------------------------------------------------------
// Bytes of one activation row of Kp elements in global memory, and the store of block b of
// a row: E4M3 32 bytes (h0, h1), E2M3 24 bytes (h0 and the first half of h1: six dwords).
template <int F>
__device__ __host__ constexpr long act_row_bytes(int Kp) { return (long)Kp / kBlock * fmt_blk_bytes<F>(); }

template <int F>
__device__ __forceinline__ void store_act_block(uint8_t* row, int b, uint4 h0, uint4 h1) {
  if constexpr (F == kFmtE2M3) {
    uint2* d = reinterpret_cast<uint2*>(row + 24L * b);  // 8-byte aligned
    d[0] = make_uint2(h0.x, h0.y);
    d[1] = make_uint2(h0.z, h0.w);
    d[2] = make_uint2(h1.x, h1.y);
  } else {
    uint4* d = reinterpret_cast<uint4*>(row + 32L * b);
    d[0] = h0;
    d[1] = h1;
  }
}

template <int TERMS>
__global__ __launch_bounds__(256) void quant_x_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                      int Hp, uint8_t* __restrict__ qhi,
                                                      uint8_t* __restrict__ qlo,
                                                      uint8_t* __restrict__ shi,
                                                      uint8_t* __restrict__ slo) {
  const int nbk = Hp / kBlock;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)T * nbk) return;
  const long t = idx / nbk;
  const int b = (int)(idx - t * nbk);
  uint4 h0 = make_uint4(0, 0, 0, 0), h1 = h0, l0 = h0, l1 = h0;
  uint32_t sh = 127, sl = 127;
  if (kBlock * b < H) {
    const uint4* src = reinterpret_cast<const uint4*>(x + t * H + kBlock * b);
    float v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 w = src[q];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * q + 2 * i] = bf16_bits_to_f32(ww[i] & 0xffffu);
        v[8 * q + 2 * i + 1] = bf16_bits_to_f32(ww[i] >> 16);
      }
    }
    if constexpr (act_fmt<TERMS>() == kFmtE2M3) {
      v6u_t hi, lo;
      mx6_encode_block(v, hi, lo, sh, sl);
      h0 = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      h1 = make_uint4(hi[4], hi[5], 0, 0);
      l0 = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      l1 = make_uint4(lo[4], lo[5], 0, 0);
    } else {
      mx8_encode_block<TERMS>(v, h0, h1, l0, l1, sh, sl);
    }
  }
  store_act_block<act_fmt<TERMS>()>(qhi + t * act_row_bytes<act_fmt<TERMS>()>(Hp), b, h0, h1);
  shi[t * nbk + b] = (uint8_t)sh;
  if constexpr (TERMS == 2) {
    store_act_block<act_fmt<TERMS>()>(qlo + t * act_row_bytes<act_fmt<TERMS>()>(Hp), b, l0, l1);
    slo[t * nbk + b] = (uint8_t)sl;
  }
}

// ---------------------------------------------------------------------------------------
// Grouped GEMM core shared by both stages. A workgroup owns one M-block (up to kBlockRows
// rows of one expert's group) and a tile of weight rows: each wave takes 6 B words per chunk
// (gate/up: 3 consecutive 16-row tiles of each matrix; down: 6 tiles of W_down), so every A
// operand read from LDS feeds 6 pairs of MFMAs. Per 128-element chunk of K:
//  * the block's A rows (hi, lo, scales) are staged in one of two LDS buffers; each thread
//    moves three (E2M3) or four (E4M3) 16-byte pieces and (threads < 2 * kBlockRows) one
//    scale dword, loaded from global memory about one chunk ahead of their store;
//  * each wave loads its B words (one 1 KB word per tile) one or two chunks ahead;
//  * 16-row subtiles past the block's rows are skipped (wave-uniform);
//  * one barrier per chunk.
// Every load is issued with a clamped chunk index, so the wait counts stay exact. Both GEMM
// kernels are held to 2 wavefronts per SIMD (6 B words, 96 accumulators and 2 B sets per
// lane; at most 256 registers), two workgroups per CU, so the other workgroup's chunks
// cover each wave's memory waits.
// ---------------------------------------------------------------------------------------
struct GemmCtx {
  const uint8_t* ahi;
  const uint8_t* alo;
  const uint8_t* ashi;
  const uint8_t* aslo;
  long r0, r1, r2, r3;  // byte offsets of the A rows of this thread's pieces (four; two hi
                        // pieces with one term)
  long sr;              // byte offset of the scale row of this thread's scale dword
  int part;             // E4M3: 16-byte piece of the row (0..7 hi, 8..15 lo), same for all
                        // pieces; E2M3: piece of the first row (0..5 hi, 6..11 lo)
  int part1, part2;     // E2M3: pieces of the second and third row
  int KB;               // K blocks of 32
  int Kp;               // row pitch of the A data, bytes
  int Ksp;              // row pitch of the A scales, bytes (padded K / 32)
};

// The staged values travel in five separate registers (d0..d3, s): a struct or array
// carried around the K loop is placed in private memory. With one term a thread moves two
// hi pieces (d0, d1) and its scale dword is the hi one (the lo slot of the LDS scale row is
// filled with the same bytes and never read).
template <int TERMS>
__device__ __forceinline__ void stage_load(const GemmCtx& cx, int c, uint4& d0, uint4& d1,
                                           uint4& d2, uint4& d3, uint32_t& sv) {
  if constexpr (act_fmt<TERMS>() == kFmtE2M3) {
    // three pieces: 96 bytes per row, chunk and term
    auto piece = [&](long r, int part) {
      const uint8_t* base = part < 6 ? cx.ahi : cx.alo;
      return *reinterpret_cast<const uint4*>(base + r + 96L * c + 16 * (part < 6 ? part : part - 6));
    };
    d0 = piece(cx.r0, cx.part);
    d1 = piece(cx.r1, cx.part1);
    d2 = piece(cx.r2, cx.part2);
  } else {
    const long off = 128L * c + 16 * (cx.part & 7);
    const uint8_t* base = cx.part < 8 ? cx.ahi : cx.alo;
    d0 = *reinterpret_cast<const uint4*>(base + cx.r0 + off);
    d1 = *reinterpret_cast<const uint4*>(base + cx.r1 + off);
    if constexpr (TERMS == 2) {
      d2 = *reinterpret_cast<const uint4*>(base + cx.r2 + off);
      d3 = *reinterpret_cast<const uint4*>(base + cx.r3 + off);
    }
  }
  const int tid = threadIdx.x;
  const uint8_t* sb = (TERMS == 2 && (tid & 1)) ? cx.aslo : cx.ashi;
  sv = *reinterpret_cast<const uint32_t*>(sb + cx.sr + 4L * c);
}

// piece i of thread tid: q = tid + kBThreads i, row q / 16, part q % 16 (two terms) or row
// q / 8, part q % 8 (one term)
template <int TERMS>
__device__ __forceinline__ void stage_store(uint8_t* lds, uint8_t* lds_s, uint4 d0, uint4 d1,
                                            uint4 d2, uint4 d3, uint32_t sv) {
  const int tid = threadIdx.x;
  if constexpr (act_fmt<TERMS>() == kFmtE2M3) {
    // piece q = tid + kBThreads i: row q / 12, part q % 12 (0..5 hi, 6..11 lo)
    constexpr int kP = fmt_pitch<kFmtE2M3>();
    auto dst = [&](int q) {
      const int row = q / 12, part = q - 12 * (q / 12);
      return lds + row * kP + (part < 6 ? 16 * part : 96 + 16 * (part - 6));
    };
    *reinterpret_cast<uint4*>(dst(tid)) = d0;
    *reinterpret_cast<uint4*>(dst(tid + kBThreads)) = d1;
    *reinterpret_cast<uint4*>(dst(tid + 2 * kBThreads)) = d2;
  } else {
    constexpr int kP = fmt_pitch<kFmtE4M3>();
    constexpr int kParts = 8 * TERMS;
    uint8_t* p = lds + (tid / kParts) * kP + 16 * (tid % kParts);
    constexpr int kRowStep = (kBThreads / kParts) * kP;
    *reinterpret_cast<uint4*>(p) = d0;
    *reinterpret_cast<uint4*>(p + kRowStep) = d1;
    if constexpr (TERMS == 2) {
      *reinterpret_cast<uint4*>(p + 2 * kRowStep) = d2;
      *reinterpret_cast<uint4*>(p + 3 * kRowStep) = d3;
    }
  }
  if (tid < 2 * kBlockRows) *reinterpret_cast<uint32_t*>(lds_s + 4 * tid) = sv;
}

// A operand (hi or lo) of 16-row subtile m for this lane; halves of K-blocks past K are
// zeroed with the lane masks m0 / m1 (all ones or zero: a select, not a branch, so the
// LDS reads of one subtile can be scheduled under the previous subtile's MFMAs).
// The A rows need no masking past K: every producer writes its rows' padding K-blocks (up to
// the next multiple of 128) as zero codes with scale byte 127, and the staging never reads
// beyond them.
__device__ __forceinline__ i32x8_t a_operand(const uint8_t* lds, int m, int lane, bool lo) {
  const int r = lane & 15, g = lane >> 4;
  const uint8_t* row = lds + (16 * m + r) * fmt_pitch<kFmtE4M3>() + (lo ? 128 : 0);
  const uint4 p0 = *reinterpret_cast<const uint4*>(row + 16 * g);
  const uint4 p1 = *reinterpret_cast<const uint4*>(row + 64 + 16 * g);
  return i32x8_t{(int)p0.x, (int)p0.y, (int)p0.z, (int)p0.w,
                 (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w};
}

// E2M3 A operand (hi or lo) of subtile m: lane 16 g + r holds row r's K-block g, its 32
// codes in six dwords (24 bytes at 24 g of the row's 96).
__device__ __forceinline__ i32x8_t a_operand6(const uint8_t* lds, int m, int lane, bool lo) {
  const int r = lane & 15, g = lane >> 4;
  const uint8_t* p = lds + (16 * m + r) * fmt_pitch<kFmtE2M3>() + (lo ? 96 : 0) + 24 * g;
  const uint2 p0 = *reinterpret_cast<const uint2*>(p);
  const uint2 p1 = *reinterpret_cast<const uint2*>(p + 8);
  const uint2 p2 = *reinterpret_cast<const uint2*>(p + 16);
  return i32x8_t{(int)p0.x, (int)p0.y, (int)p1.x, (int)p1.y, (int)p2.x, (int)p2.y, 0, 0};
}

__device__ __forceinline__ i32x8_t b_operand(uint4 w) {
  return i32x8_t{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
}

// One B word for this lane: 16 code bytes and the scale byte. Past K the lane reads another
// word of the tile and its values are not masked here: a select at load time would wait for
// the load at once (every chunk would then wait for the B loads it has just issued). They
// need no masking: the A data of those K blocks is zero, FP4 codes are finite, and the
// scale is replaced by 1 where it is used (a NaN scale byte would poison the zero products).
// Tiles past the matrix rows read the last tile; their columns are never stored.
struct BWord {
  uint4 w;
  uint32_t s;
};

template <bool NT>
__device__ __forceinline__ BWord load_b(const uint8_t* codes, const uint8_t* scales, int c,
                                        int KB) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const long w = (4 * c + g < KB) ? 64L * c + lane : 64L * c;  // past K: any valid word
  BWord b;
  b.w = ld_w16<NT>(codes + 16 * w);
  b.s = scales[w];
  return b;
}

// The B words of one wave: NB = (matrices) x kNS tiles, word q = matrix * kNS + tile. Named
// members (an array carried around the K loop would be placed in private memory).
struct BPtrs {
  const uint8_t *c0, *c1, *c2, *c3, *c4, *c5;  // code base of word q (tile-major word 0)
  const uint8_t *s0, *s1, *s2, *s3, *s4, *s5;  // scale base of word q
  bool on0;                                    // the wave's first tile lies inside its matrix
};

template <int NB>
struct BSet {
  BWord w0, w1, w2, w3, w4, w5;
};

template <int NB, bool NT>
__device__ __forceinline__ BSet<NB> load_bset(const BPtrs& p, int c, int KB) {
  BSet<NB> r;
  r.w0 = load_b<NT>(p.c0, p.s0, c, KB);
  r.w1 = r.w2 = r.w3 = r.w4 = r.w5 = r.w0;
  if constexpr (NB > 1) r.w1 = load_b<NT>(p.c1, p.s1, c, KB);
  if constexpr (NB > 2) r.w2 = load_b<NT>(p.c2, p.s2, c, KB);
  if constexpr (NB > 3) r.w3 = load_b<NT>(p.c3, p.s3, c, KB);
  if constexpr (NB > 4) r.w4 = load_b<NT>(p.c4, p.s4, c, KB);
  if constexpr (NB > 5) r.w5 = load_b<NT>(p.c5, p.s5, c, KB);
  return r;
}

// acc[m][q] accumulates 16-row subtile m against B word q.
template <int NB>
struct Acc {
  f32x4_t a[kMSub][NB];
};

// sb: the B word's scale byte, or 127 (scale 1) past K. F: the A operand's format code.
template <int F>
__device__ __forceinline__ void mfma2(f32x4_t& acc, const i32x8_t& ahi, const i32x8_t& alo,
                                      const BWord& b, int sw_hi, int sw_lo, int sb) {
  const i32x8_t bq = b_operand(b.w);
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ahi, bq, acc, F, 4, 0, sw_hi, 0, sb);
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(alo, bq, acc, F, 4, 0, sw_lo, 0, sb);
}

template <int F>
__device__ __forceinline__ void mfma1(f32x4_t& acc, const i32x8_t& ahi, const BWord& b, int sw_hi,
                                      int sb) {
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ahi, b_operand(b.w), acc, F, 4, 0, sw_hi, 0, sb);
}

// The MFMAs of one chunk: for each 16-row subtile m of the block (those holding rows), its
// A operand (hi, and lo with two terms) and scale bytes from LDS against the wave's NB B
// words. With MOE_FP4_A_PIPE (two terms) the LDS reads run under MFMAs without more
// registers: lo of m is read before the hi MFMAs of m are issued, hi of m + 1 before the
// lo MFMAs of m.
#ifndef MOE_FP4_A_PIPE
#define MOE_FP4_A_PIPE 1
#endif
template <int F, int TERMS>
struct AOperand {
  i32x8_t hi, lo;
  int sh, sl;
};

template <int F, int TERMS>
__device__ __forceinline__ AOperand<F, TERMS> load_a_operand(const uint8_t* A, const uint8_t* AS,
                                                             int m, int lane) {
  const int r = lane & 15, g = lane >> 4;
  AOperand<F, TERMS> o;
  o.hi = F == kFmtE2M3 ? a_operand6(A, m, lane, false) : a_operand(A, m, lane, false);
  o.sh = (int)AS[8 * (16 * m + r) + g];
  if constexpr (TERMS == 2) {
    o.lo = F == kFmtE2M3 ? a_operand6(A, m, lane, true) : a_operand(A, m, lane, true);
    o.sl = (int)AS[8 * (16 * m + r) + 4 + g];
  } else {
    o.lo = o.hi;
    o.sl = o.sh;
  }
  return o;
}

template <int F, int NB, int TERMS>
__device__ __forceinline__ void subtile_mfmas(f32x4_t (&a)[NB], const AOperand<F, TERMS>& o,
                                              const BSet<NB>& BS, bool s_ok) {
  // past K the B lanes read another word: its scale byte is replaced by 1 (127)
  const int sb0 = s_ok ? (int)BS.w0.s : 127, sb1 = s_ok ? (int)BS.w1.s : 127;
  const int sb2 = s_ok ? (int)BS.w2.s : 127, sb3 = s_ok ? (int)BS.w3.s : 127;
  const int sb4 = s_ok ? (int)BS.w4.s : 127, sb5 = s_ok ? (int)BS.w5.s : 127;
  if constexpr (TERMS == 2) {
    mfma2<F>(a[0], o.hi, o.lo, BS.w0, o.sh, o.sl, sb0);
    if constexpr (NB > 1) mfma2<F>(a[1], o.hi, o.lo, BS.w1, o.sh, o.sl, sb1);
    if constexpr (NB > 2) mfma2<F>(a[2], o.hi, o.lo, BS.w2, o.sh, o.sl, sb2);
    if constexpr (NB > 3) mfma2<F>(a[3], o.hi, o.lo, BS.w3, o.sh, o.sl, sb3);
    if constexpr (NB > 4) mfma2<F>(a[4], o.hi, o.lo, BS.w4, o.sh, o.sl, sb4);
    if constexpr (NB > 5) mfma2<F>(a[5], o.hi, o.lo, BS.w5, o.sh, o.sl, sb5);
  } else {
    mfma1<F>(a[0], o.hi, BS.w0, o.sh, sb0);
    if constexpr (NB > 1) mfma1<F>(a[1], o.hi, BS.w1, o.sh, sb1);
    if constexpr (NB > 2) mfma1<F>(a[2], o.hi, BS.w2, o.sh, sb2);
    if constexpr (NB > 3) mfma1<F>(a[3], o.hi, BS.w3, o.sh, sb3);
    if constexpr (NB > 4) mfma1<F>(a[4], o.hi, BS.w4, o.sh, sb4);
    if constexpr (NB > 5) mfma1<F>(a[5], o.hi, BS.w5, o.sh, sb5);
  }
}

// One term's MFMAs of one subtile: the accumulators a against the NB B words.
template <int F, int NB>
__device__ __forceinline__ void term_mfmas(f32x4_t (&a)[NB], const i32x8_t& op, int sw,
                                           const BSet<NB>& BS, bool s_ok) {
  const int sb0 = s_ok ? (int)BS.w0.s : 127, sb1 = s_ok ? (int)BS.w1.s : 127;
  const int sb2 = s_ok ? (int)BS.w2.s : 127, sb3 = s_ok ? (int)BS.w3.s : 127;
  const int sb4 = s_ok ? (int)BS.w4.s : 127, sb5 = s_ok ? (int)BS.w5.s : 127;
  mfma1<F>(a[0], op, BS.w0, sw, sb0);
  if constexpr (NB > 1) mfma1<F>(a[1], op, BS.w1, sw, sb1);
  if constexpr (NB > 2) mfma1<F>(a[2], op, BS.w2, sw, sb2);
  if constexpr (NB > 3) mfma1<F>(a[3], op, BS.w3, sw, sb3);
  if constexpr (NB > 4) mfma1<F>(a[4], op, BS.w4, sw, sb4);
  if constexpr (NB > 5) mfma1<F>(a[5], op, BS.w5, sw, sb5);
}

template <int F>
__device__ __forceinline__ i32x8_t a_term(const uint8_t* A, int m, int lane, bool lo) {
  return F == kFmtE2M3 ? a_operand6(A, m, lane, lo) : a_operand(A, m, lane, lo);
}

template <int F, int NB, int TERMS>
__device__ __forceinline__ void chunk_mfmas(const uint8_t* A, const uint8_t* AS, int rows, int lane,
                                            const BSet<NB>& BS, bool s_ok, Acc<NB>& acc) {
  if constexpr (MOE_FP4_A_PIPE && TERMS == 2) {
    const int r = lane & 15, g = lane >> 4;
    i32x8_t hi = a_term<F>(A, 0, lane, false);
    int sh = (int)AS[8 * r + g];
#pragma unroll
    for (int m = 0; m < kMSub; ++m) {
      if (16 * m < rows) {  // wave-uniform
        const i32x8_t lo = a_term<F>(A, m, lane, true);
        const int sl = (int)AS[8 * (16 * m + r) + 4 + g];
        term_mfmas<F, NB>(acc.a[m], hi, sh, BS, s_ok);
        if (m + 1 < kMSub) {
          hi = a_term<F>(A, m + 1, lane, false);
          sh = (int)AS[8 * (16 * (m + 1) + r) + g];
        }
        term_mfmas<F, NB>(acc.a[m], lo, sl, BS, s_ok);
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < kMSub; ++m) {
      if (16 * m < rows) {  // wave-uniform
        const AOperand<F, TERMS> o = load_a_operand<F, TERMS>(A, AS, m, lane);
        subtile_mfmas<F, NB, TERMS>(acc.a[m], o, BS, s_ok);
      }
    }
  }
}

// BSETS 2 or 3: the K loop runs BSETS chunks per trip with BSETS B sets used in turn and
// reloaded in place, BSETS chunks ahead (gate/up, which has the registers for it). BSETS 1:
// one B set rotates (current = next), a register copy that waits for the next set's loads,
// two chunks ahead; the smaller register budget of down keeps it spill-free.
// ADEPTH 2 (with BSETS 2): the A staging loads run two chunks ahead of their LDS store, in
// two register sets used on alternate chunks (no copies between them).
// TERMS 1: the A rows hold one MXFP8 term (hi), one MFMA per B word. TERMS 2: two terms of
// the two-term format (E2M3 by default).
template <int NB, int BSETS, int ADEPTH, int TERMS, bool NT>
__device__ __forceinline__ void gemm_k_loop(const GemmCtx& cx, const BPtrs& bp, int rows,
                                            uint8_t* lds, uint8_t* lds_s, Acc<NB>& acc) {
  static_assert(ADEPTH == 1 || (ADEPTH == 2 && BSETS == 2), "A depth 2 runs with two B sets");
  constexpr bool PAIR = BSETS > 1;
  static_assert(BSETS >= 1 && BSETS <= 3, "B sets");
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int nch = (cx.KB + 3) / 4;
  constexpr int F = act_fmt<TERMS>();
  constexpr int kBuf = kBlockRows * fmt_pitch<F>();
  constexpr int kBufS = kBlockRows * 8;
  uint4 d0, d1, d2, d3, e0, e1, e2, e3;
  uint32_t sv, se;
  stage_load<TERMS>(cx, 0, d0, d1, d2, d3, sv);
  stage_store<TERMS>(lds, lds_s, d0, d1, d2, d3, sv);
  stage_load<TERMS>(cx, min(1, nch - 1), d0, d1, d2, d3, sv);
  if constexpr (ADEPTH == 2) stage_load<TERMS>(cx, min(2, nch - 1), e0, e1, e2, e3, se);
  // B sets: chunk c uses b[c % BSETS] (BSETS > 1) or the rotated pair b0 <- b1
  BSet<NB> b0 = load_bset<NB, NT>(bp, 0, cx.KB);
  BSet<NB> b1 = load_bset<NB, NT>(bp, min(1, nch - 1), cx.KB);
  BSet<NB> b2 = b1;
  if constexpr (BSETS == 3) b2 = load_bset<NB, NT>(bp, min(2, nch - 1), cx.KB);
  const bool any_on = bp.on0;  // tile 0 of matrix 0 is the wave's first tile
  __syncthreads();
  // One chunk C with B set BS: MFMAs on the A buffer of C, then A of C + 1 into the other
  // buffer (last read in chunk C - 1, before its barrier), the A loads of C + 2, the B loads
  // of C + 2 into BS (clamped), one barrier. A halves of this lane: K-blocks
  // 4 C + 2 h + g / 2 (E4M3) or 4 C + g (E2M3); its scale: K-block 4 C + g. Past K the A rows
  // hold zero codes with scale byte 127 (written by their producers), and the B scale is
  // forced to 1: the B lanes there read another word, whose scale byte may be 255 (NaN),
  // which would poison the zero products.
#define MOE_FP4_KSTEP(C, BS, X0, X1, X2, X3, XS)                                                 \
  {                                                                                             \
    const uint8_t* A = lds + ((C) & 1) * kBuf;                                                  \
    const uint8_t* AS = lds_s + ((C) & 1) * kBufS;                                              \
    const bool s_ok = 4 * (C) + g < cx.KB;                                                      \
    if (any_on) chunk_mfmas<F, NB, TERMS>(A, AS, rows, lane, BS, s_ok, acc);                     \
    stage_store<TERMS>(lds + (((C) + 1) & 1) * kBuf, lds_s + (((C) + 1) & 1) * kBufS, X0, X1,   \
                       X2, X3, XS);                                                             \
    const int cn = min((C) + 2, nch - 1);                                                       \
    stage_load<TERMS>(cx, min((C) + 1 + ADEPTH, nch - 1), X0, X1, X2, X3, XS);                  \
    if constexpr (PAIR) {                                                                       \
      /* the A loads go out before the B loads, so the next LDS store waits for A only */       \
      __builtin_amdgcn_sched_barrier(0);                                                        \
      BS = load_bset<NB, NT>(bp, min((C) + BSETS, nch - 1), cx.KB);                             \
    } else {                                                                                    \
      b0 = b1;                                                                                  \
      b1 = load_bset<NB, NT>(bp, cn, cx.KB);                                                    \
    }                                                                                           \
    __syncthreads();                                                                            \
  }
  // the pair loop has no condition inside, so both B sets keep their registers across the
  // back edge (a conditional second step makes the compiler copy them, which waits for
  // their loads); an odd last chunk runs after it
  if constexpr (BSETS == 3) {
    int c = 0;
    for (; c + 2 < nch; c += 3) {
      MOE_FP4_KSTEP(c, b0, d0, d1, d2, d3, sv)
      MOE_FP4_KSTEP(c + 1, b1, d0, d1, d2, d3, sv)
      MOE_FP4_KSTEP(c + 2, b2, d0, d1, d2, d3, sv)
    }
    if (c < nch) MOE_FP4_KSTEP(c, b0, d0, d1, d2, d3, sv)
    if (c + 1 < nch) MOE_FP4_KSTEP(c + 1, b1, d0, d1, d2, d3, sv)
  } else if constexpr (BSETS == 2 && ADEPTH == 2) {
    int c = 0;
    for (; c + 1 < nch; c += 2) {
      MOE_FP4_KSTEP(c, b0, d0, d1, d2, d3, sv)
      MOE_FP4_KSTEP(c + 1, b1, e0, e1, e2, e3, se)
    }
    if (c < nch) MOE_FP4_KSTEP(c, b0, d0, d1, d2, d3, sv)
  } else if constexpr (BSETS == 2) {
    int c = 0;
    for (; c + 1 < nch; c += 2) {
      MOE_FP4_KSTEP(c, b0, d0, d1, d2, d3, sv)
      MOE_FP4_KSTEP(c + 1, b1, d0, d1, d2, d3, sv)
    }
    if (c < nch) MOE_FP4_KSTEP(c, b0, d0, d1, d2, d3, sv)
  } else {
    for (int c = 0; c < nch; ++c) MOE_FP4_KSTEP(c, b0, d0, d1, d2, d3, sv)
  }

#undef MOE_FP4_KSTEP
}

// Fills the per-thread A row offsets. row_of(i) returns the A row (token or sorted position)
// of block row i (clamped into the block by the caller).
template <int TERMS, typename RowOf>
__device__ __forceinline__ void gemm_ctx_rows(GemmCtx& cx, RowOf row_of) {
  const int tid = threadIdx.x;
  if constexpr (act_fmt<TERMS>() == kFmtE2M3) {
    // 12 pieces per row (6 hi, 6 lo), pieces tid, tid + 256, tid + 512 of the 768
    static_assert(kBlockRows * 12 == 3 * kBThreads, "pieces cover the block's rows");
    cx.r0 = (long)row_of(tid / 12) * cx.Kp;
    cx.r1 = (long)row_of((tid + kBThreads) / 12) * cx.Kp;
    cx.r2 = (long)row_of((tid + 2 * kBThreads) / 12) * cx.Kp;
    cx.r3 = cx.r0;
    cx.part = tid % 12;
    cx.part1 = (tid + kBThreads) % 12;
    cx.part2 = (tid + 2 * kBThreads) % 12;
  } else {
    constexpr int kParts = 8 * TERMS;              // 16-byte pieces per staged row
    constexpr int kRows = kBThreads / kParts;      // rows covered by one piece index
    static_assert(kRows * (2 * TERMS) == kBlockRows, "pieces cover the block's rows");
    cx.r0 = (long)row_of(tid / kParts) * cx.Kp;
    cx.r1 = (long)row_of(tid / kParts + kRows) * cx.Kp;
    cx.r2 = cx.r3 = cx.r0;
    if constexpr (TERMS == 2) {
      cx.r2 = (long)row_of(tid / kParts + 2 * kRows) * cx.Kp;
      cx.r3 = (long)row_of(tid / kParts + 3 * kRows) * cx.Kp;
    }
    cx.part = tid % kParts;
    cx.part1 = cx.part2 = cx.part;
  }
  cx.sr = (long)row_of(min(tid >> 1, kBlockRows - 1)) * cx.Ksp;
}

// Workgroup -> (row block, column tile). The dispatcher hands workgroups to the eight XCDs
// in turn (b mod 8) and each XCD has its own L2, so the logical index L gives every XCD one
// contiguous range of the n_blocks x n_tiles items (sized from the actual block count, so
// the XCDs get equal shares). L runs over groups of up to kGroupBlocks row blocks of one
// expert (a group starts at the expert's first block, the next kGroupBlocks blocks later);
// inside a group the column tiles go in order and the group's row blocks run fastest. The
// row blocks that read one weight tile are adjacent in time on one XCD, and a row block's
// activation rows are read again for each column tile a group's width later, while they
// are still in that L2: weights and activations both come from HBM about once. The item's
// expert, first sorted row and row count are returned; false for the workgroups past the
// items (the grid is nb_max x n_tiles rounded up to a multiple of 8).
constexpr int kXcds = 8;
#ifndef MOE_FP4_GROUP_BLOCKS
#define MOE_FP4_GROUP_BLOCKS 8  // row blocks of one expert whose items are interleaved
#endif
constexpr int kGroupBlocks = MOE_FP4_GROUP_BLOCKS;

__device__ __forceinline__ bool map_block_tile(int b, int nb, int n_tiles,
                                               const int32_t* __restrict__ blk_expert,
                                               const int32_t* __restrict__ blk_row0,
                                               const int32_t* __restrict__ offsets, int& e,
                                               int& row0, int& rows, int& nt) {
  const long G = (long)nb * n_tiles;
  const long per = (G + kXcds - 1) / kXcds;
  const int j = b / kXcds;
  if (j >= per) return false;
  const long L = (long)(b - j * kXcds) * per + j;
  if (L >= G) return false;
  const int bl = (int)(L / n_tiles);  // a row block of the item's group
  e = blk_expert[bl];
  const int o0 = offsets[e];
  const int n = offsets[e + 1] - o0;  // the expert's sorted rows
  const int jb = (blk_row0[bl] - o0) / kBlockRows;  // bl's index among the expert's blocks
  const int g0 = jb / kGroupBlocks * kGroupBlocks;
  const int ng = min(kGroupBlocks, (n + kBlockRows - 1) / kBlockRows - g0);
  const long local = L - (long)(bl - jb + g0) * n_tiles;  // in [0, ng x n_tiles)
  nt = (int)(local / ng);
  const int jj = g0 + (int)(local - (long)nt * ng);
  row0 = o0 + jj * kBlockRows;
  rows = min(kBlockRows, n - jj * kBlockRows);
  return true;
}

// ---------------------------------------------------------------------------------------
// 3. gate / up / SiLU / h quantisation
// ---------------------------------------------------------------------------------------
template <int TERMS, bool NT>
__global__ __launch_bounds__(kBThreads) __attribute__((amdgpu_waves_per_eu(MOE_FP4_GU_WPE))) void gemm_gate_up_kernel(
    const uint8_t* __restrict__ xhi, const uint8_t* __restrict__ xlo,
    const uint8_t* __restrict__ xshi, const uint8_t* __restrict__ xslo, int Hp,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ blk_expert,
    const int32_t* __restrict__ blk_row0, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ n_blocks, int k, const uint8_t* __restrict__ packed,
    size_t stride, size_t off_gc, size_t off_uc, size_t off_gs, size_t off_us, int H, int I,
    int n_tiles, uint8_t* __restrict__ hhi, uint8_t* __restrict__ hlo,
    uint8_t* __restrict__ hshi, uint8_t* __restrict__ hslo, int Ip) {
  constexpr int F = act_fmt<TERMS>();
  // epilogue h tile over the A buffers: row r's 32-block b at r * kHP + kHBP * b (fp32). With
  // 36-float blocks and a row pitch of 24 mod 64 floats, the sixteen 16-byte reads served
  // together fall on distinct banks (a 193-float pitch had 8-way conflicts) and the
  // accumulator stores are at most 2-way.
  constexpr int kHBP = 36;
  constexpr int kHP = (kBN / 32) * kHBP + ((24 - (kBN / 32) * kHBP) % 64 + 64) % 64;
  __shared__ __align__(16) uint8_t lds[std::max(2 * kBlockRows * fmt_pitch<F>(), kBlockRows * kHP * 4)];
  __shared__ __align__(16) uint8_t lds_s[2 * kBlockRows * 8];
  int e, row0, rows, nt;
  if (!map_block_tile((int)blockIdx.x, n_blocks[0], n_tiles, blk_expert, blk_row0, offsets, e, row0,
                      rows, nt))
    return;  // workgroup-uniform
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int KB = H / kBlock;
  const int tile0 = (nt * kBWaves + wv) * kNS;  // first 16-row tile of gate / up of this wave

  GemmCtx cx;
  cx.ahi = xhi;
  cx.alo = xlo;
  cx.ashi = xshi;
  cx.aslo = xslo;
  cx.KB = KB;
  cx.Kp = (int)act_row_bytes<F>(Hp);
  cx.Ksp = Hp / kBlock;
  gemm_ctx_rows<TERMS>(cx, [&](int i) { return perm[row0 + min(i, rows - 1)] / k; });

  const uint8_t* base = packed + (size_t)e * stride;
  const int nt16 = I / 16;
  // word j < kNS: gate tile tile0 + j; word kNS + j: up tile tile0 + j (tile-major word index
  // tb(j); tiles past the matrix read its last tile)
  auto tb = [&](int j) { return (size_t)min(tile0 + j, nt16 - 1) * 16 * KB; };
  BPtrs bp;
  bp.c0 = base + off_gc + 16 * tb(0);
  bp.s0 = base + off_gs + tb(0);
  bp.c1 = base + (kNS > 1 ? off_gc + 16 * tb(1) : off_uc + 16 * tb(0));
  bp.s1 = base + (kNS > 1 ? off_gs + tb(1) : off_us + tb(0));
  bp.c2 = base + (kNS > 2 ? off_gc + 16 * tb(2) : off_uc + 16 * tb(2 - kNS));
  bp.s2 = base + (kNS > 2 ? off_gs + tb(2) : off_us + tb(2 - kNS));
  bp.c3 = base + off_uc + 16 * tb(3 - kNS);
  bp.s3 = base + off_us + tb(3 - kNS);
  bp.c4 = base + off_uc + 16 * tb(4 - kNS);
  bp.s4 = base + off_us + tb(4 - kNS);
  bp.c5 = base + off_uc + 16 * tb(5 - kNS);
  bp.s5 = base + off_us + tb(5 - kNS);
  bp.on0 = tile0 < nt16;
  Acc<2 * kNS> acc;
#pragma unroll
  for (int m = 0; m < kMSub; ++m)
#pragma unroll
    for (int q = 0; q < 2 * kNS; ++q) acc.a[m][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  gemm_k_loop<2 * kNS, MOE_FP4_GU_BSETS, MOE_FP4_GU_ADEPTH, TERMS, NT>(cx, bp, rows, lds, lds_s, acc);

  // epilogue: h (fp32) for the block's rows x kBN columns into LDS (the loop ended with a
  // barrier), then per (row, 32-block) quantisation by one thread
  float* htile = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int m = 0; m < kMSub; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 16 * m + 4 * (lane >> 4) + q;  // block row
#pragma unroll
      for (int j = 0; j < kNS; ++j) {  // tile tile0 + j: columns 16 j .. 16 j + 15 of the wave's
        const int col = 16 * (kNS * wv + j) + (lane & 15);
        htile[i * kHP + kHBP * (col >> 5) + (col & 31)] = silu_f32(acc.a[m][j][q]) * acc.a[m][kNS + j][q];
      }
    }
  __syncthreads();
  // one (row, 32-block) per thread and round
  for (int it = tid; it < kBlockRows * (kBN / 32); it += kBThreads) {
    const int r = it / (kBN / 32), b = it % (kBN / 32);
    const int col = nt * kBN + 32 * b;  // first I index of this 32-block
    if (r < rows && col < I) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = htile[r * kHP + kHBP * b + i];
      uint4 h0, h1, l0, l1;
      uint32_t sh, sl;
      if constexpr (F == kFmtE2M3) {
        v6u_t hi, lo;
        mx6_encode_block(v, hi, lo, sh, sl);
        h0 = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        h1 = make_uint4(hi[4], hi[5], 0, 0);
        l0 = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        l1 = make_uint4(lo[4], lo[5], 0, 0);
      } else {
        mx8_encode_block<TERMS>(v, h0, h1, l0, l1, sh, sl);
      }
      const long pos = row0 + r;
      const long rb = pos * act_row_bytes<F>(Ip);
      store_act_block<F>(hhi + rb, col / kBlock, h0, h1);
      hshi[pos * (Ip / kBlock) + col / kBlock] = (uint8_t)sh;
      if constexpr (TERMS == 2) {
        store_act_block<F>(hlo + rb, col / kBlock, l0, l1);
        hslo[pos * (Ip / kBlock) + col / kBlock] = (uint8_t)sl;
      }
    }
  }
  // the row padding I .. Ip (K-blocks of the down GEMM's last chunk past I): zero codes and
  // scale byte 127, written once per row by the last column tile's workgroup
  if (nt == n_tiles - 1) {
    const int pad = (Ip - I) / kBlock;  // 0..3 blocks
    const uint4 z = make_uint4(0, 0, 0, 0);
    for (int it = tid; it < rows * pad; it += kBThreads) {
      const int r = it / pad, b = I / kBlock + (it - (it / pad) * pad);
      const long pos = row0 + r;
      const long rb = pos * act_row_bytes<F>(Ip);
      store_act_block<F>(hhi + rb, b, z, z);
      hshi[pos * (Ip / kBlock) + b] = 127;
      if constexpr (TERMS == 2) {
        store_act_block<F>(hlo + rb, b, z, z);
        hslo[pos * (Ip / kBlock) + b] = 127;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// 4. down projection, times the router weight, fp32 per pair
// ---------------------------------------------------------------------------------------
template <int TERMS, bool NT>
__global__ __launch_bounds__(kBThreads) __attribute__((amdgpu_waves_per_eu(MOE_FP4_DN_WPE))) void gemm_down_kernel(
    const uint8_t* __restrict__ hhi, const uint8_t* __restrict__ hlo,
    const uint8_t* __restrict__ hshi, const uint8_t* __restrict__ hslo, int Ip,
    const int32_t* __restrict__ perm, const float* __restrict__ wts,
    const int32_t* __restrict__ blk_expert, const int32_t* __restrict__ blk_row0,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ n_blocks,
    const uint8_t* __restrict__ packed, size_t stride, size_t off_dc, size_t off_ds, int H, int I,
    int n_tiles, float* __restrict__ ypair) {
  constexpr int F = act_fmt<TERMS>();
  __shared__ __align__(16) uint8_t lds[2 * kBlockRows * fmt_pitch<F>()];
  __shared__ __align__(16) uint8_t lds_s[2 * kBlockRows * 8];
  int e, row0, rows, nt;
  if (!map_block_tile((int)blockIdx.x, n_blocks[0], n_tiles, blk_expert, blk_row0, offsets, e, row0,
                      rows, nt))
    return;  // workgroup-uniform
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int KB = I / kBlock;
  const int tile0 = (nt * kBWaves + wv) * kDNS;  // first 16-row tile of down (rows of H)

  GemmCtx cx;
  cx.ahi = hhi;
  cx.alo = hlo;
  cx.ashi = hshi;
  cx.aslo = hslo;
  cx.KB = KB;
  cx.Kp = (int)act_row_bytes<F>(Ip);
  cx.Ksp = Ip / kBlock;
  gemm_ctx_rows<TERMS>(cx, [&](int i) { return row0 + min(i, rows - 1); });

  const uint8_t* base = packed + (size_t)e * stride;
  const int nt16 = H / 16;
  // word j: tile tile0 + j (tile-major word index tb(j); tiles past H read the last tile)
  auto tb = [&](int j) { return (size_t)min(tile0 + j, nt16 - 1) * 16 * KB; };
  BPtrs bp;
  bp.c0 = base + off_dc + 16 * tb(0);
  bp.c1 = base + off_dc + 16 * tb(1);
  bp.c2 = base + off_dc + 16 * tb(2);
  bp.c3 = base + off_dc + 16 * tb(3);
  bp.c4 = base + off_dc + 16 * tb(4);
  bp.c5 = base + off_dc + 16 * tb(5);
  bp.s0 = base + off_ds + tb(0);
  bp.s1 = base + off_ds + tb(1);
  bp.s2 = base + off_ds + tb(2);
  bp.s3 = base + off_ds + tb(3);
  bp.s4 = base + off_ds + tb(4);
  bp.s5 = base + off_ds + tb(5);
  bp.on0 = tile0 < nt16;
  Acc<kDNS> acc;
#pragma unroll
  for (int m = 0; m < kMSub; ++m)
#pragma unroll
    for (int q = 0; q < kDNS; ++q) acc.a[m][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  gemm_k_loop<kDNS, MOE_FP4_DN_BSETS, 1, TERMS, NT>(cx, bp, rows, lds, lds_s, acc);

  // per block row: its pair and router weight once, then the wave's tiles
#pragma unroll
  for (int m = 0; m < kMSub; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 16 * m + 4 * (lane >> 4) + q;
      if (i < rows) {
        const int pair = perm[row0 + i];
        const float wp = wts[pair];
        float* yrow = ypair + (size_t)pair * H + (lane & 15);
#pragma unroll
        for (int s2 = 0; s2 < kDNS; ++s2)
          if (tile0 + s2 < nt16) yrow[16 * (tile0 + s2)] = wp * acc.a[m][s2][q];
      }
    }
}

// ---------------------------------------------------------------------------------------
// 5. combine: workgroup = one token x kCombineCols columns, four consecutive columns per
// thread. Every thread ranks the token's slots itself (the ids and weights are the same
// for the whole workgroup), so the k row loads are issued together, before the ranks are
// known, and summed afterwards in canonical order: ascending expert id, then weight bits,
// then slot; invalid ids dropped.
// ---------------------------------------------------------------------------------------
constexpr int kCombineCols = 4 * 256;

__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ ids,
                                                      const float* __restrict__ wts, int k,
                                                      int n_experts, int H, int col_blocks,
                                                      const float* __restrict__ ypair,
                                                      uint16_t* __restrict__ y) {
  const int t = blockIdx.x / col_blocks;
  const int n0 = (blockIdx.x - t * col_blocks) * kCombineCols + 4 * threadIdx.x;
  const bool col_ok = n0 < H;
  // lane j < k of every wave: slot j's id, weight bits and rank among the valid slots
  const int lane = threadIdx.x & 63;
  const int jl = min(lane, k - 1);
  const int e_l = ids[(size_t)t * k + jl];
  const uint32_t w_l = __float_as_uint(wts[(size_t)t * k + jl]);
  // the k row loads, issued before the ranks are known; unconditional, at clamped slots
  // and columns (rows of invalid slots are loaded but never summed)
  const int nc = min(n0, H - 4);
  float vx[kMaxK], vy[kMaxK], vz[kMaxK], vw[kMaxK];  // one array per component
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    const float4 r = *reinterpret_cast<const float4*>(ypair + ((size_t)t * k + min(j, k - 1)) * H + nc);
    vx[j] = r.x;
    vy[j] = r.y;
    vz[j] = r.z;
    vw[j] = r.w;
  }
  // one wait for all the loads above; keeps the row loads here rather than in the sum
  int e_r = e_l;
  uint32_t w_r = w_l;
  asm volatile("" : "+v"(e_r), "+v"(w_r));
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) asm volatile("" : "+v"(vx[j]), "+v"(vy[j]), "+v"(vz[j]), "+v"(vw[j]));

  const bool ok_l = lane < k && e_r >= 0 && e_r < n_experts;
  const unsigned long long okm = __ballot(ok_l);  // every lane votes
  int rank = 0;
  for (int i = 0; i < k; ++i) {
    const int ei = __builtin_amdgcn_readlane(e_r, i);
    const uint32_t wi = (uint32_t)__builtin_amdgcn_readlane((int)w_r, i);
    const bool before = ei < e_r || (ei == e_r && (wi < w_r || (wi == w_r && i < lane)));
    rank += (((okm >> i) & 1ull) && before) ? 1 : 0;
  }
  // order: the slot of rank p in bits 4p..4p+3
  uint32_t order = 0;
  for (int j = 0; j < k; ++j)
    if ((okm >> j) & 1ull) order |= (uint32_t)j << (4 * __builtin_amdgcn_readlane(rank, j));
  const int nv = __popcll(okm);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p = 0; p < nv; ++p) {
    const int j = (int)((order >> (4 * p)) & 15u);
    acc.x += vx[j];
    acc.y += vy[j];
    acc.z += vz[j];
    acc.w += vw[j];
  }
  if (col_ok) {
    const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc.x) | ((uint32_t)f32_to_bf16_rne(acc.y) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc.z) | ((uint32_t)f32_to_bf16_rne(acc.w) << 16);
    *reinterpret_cast<uint2*>(y + (size_t)t * H + n0) = make_uint2(lo, hi);
  }
}

// Debug: x quantised as the grouped path does it, decoded back to fp32: out[t][h] = the sum
// of the terms, each E4M3 code times 2^(scale - 127) (exact in fp32: a term has at most four
// significant bits and the two terms of a block are a few binades apart).
template <int TERMS>
__global__ __launch_bounds__(256) void dequant_act_kernel(const uint8_t* __restrict__ qhi,
                                                          const uint8_t* __restrict__ qlo,
                                                          const uint8_t* __restrict__ shi,
                                                          const uint8_t* __restrict__ slo, int T,
                                                          int H, int Hp, float* __restrict__ out) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)T * H) return;
  const long t = idx / H;
  const int h = (int)(idx - t * H);
  const long sb = t * (Hp / kBlock) + h / kBlock;
  float r;
  if constexpr (act_fmt<TERMS>() == kFmtE2M3) {
    // code h % 32 of the block's six dwords
    const long rb = t * act_row_bytes<kFmtE2M3>(Hp) + 24L * (h / kBlock);
    const uint32_t* wh = reinterpret_cast<const uint32_t*>(qhi + rb);
    const uint32_t* wl = reinterpret_cast<const uint32_t*>(qlo + rb);
    v6u_t vh, vl;
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      vh[i] = wh[i];
      vl[i] = wl[i];
    }
    const int i = h % kBlock;
    r = e2m3_value(e2m3_code(vh, i), (int)shi[sb] - 127) + e2m3_value(e2m3_code(vl, i), (int)slo[sb] - 127);
  } else {
    r = ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)qhi[t * Hp + h], 0), (int)shi[sb] - 127);
    if constexpr (TERMS == 2)
      r += ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)qlo[t * Hp + h], 0), (int)slo[sb] - 127);
  }
  out[idx] = r;
}

template <int TERMS>
hipError_t debug_act_quant(const uint16_t* x, int T, int H, uint8_t* ws, float* out, hipStream_t s) {
  const int Hp = (H + 127) / 128 * 128;
  const size_t q = (size_t)T * Hp, sc = (size_t)T * (Hp / kBlock);
  uint8_t *qhi = ws, *qlo = ws + q, *shi = ws + 2 * q, *slo = ws + 2 * q + sc;
  const long qn = (long)T * (Hp / kBlock);
  hipError_t e = launch_kernel(kKindBatchedQuant, quant_x_kernel<TERMS>,
                               dim3((unsigned)((qn + 255) / 256)), dim3(256), 0, s, x, T, H, Hp, qhi,
                               qlo, shi, slo);
  if (e != hipSuccess) return e;
  const long n = (long)T * H;
  return launch_kernel(kKindBatchedQuant, dequant_act_kernel<TERMS>, dim3((unsigned)((n + 255) / 256)),
                       dim3(256), 0, s, qhi, qlo, shi, slo, T, H, Hp, out);
}

}  // namespace

BatchedLayout batched_layout(int T, int k, int n_experts, int hidden, int inter) {
  BatchedLayout L{};
  const size_t P = (size_t)T * (size_t)k;
  const size_t Hp = (size_t)((hidden + 127) / 128) * 128;
  const size_t Ip = (size_t)((inter + 127) / 128) * 128;
  const size_t nb_max = (P + kBlockRows - 1) / kBlockRows + (size_t)n_experts;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  L.offsets = take(((size_t)n_experts + 1) * 4);
  L.perm = take(P * 4);
  L.blk_expert = take(nb_max * 4);
  L.blk_row0 = take(nb_max * 4);
  L.n_blocks = take(4);
  L.sort_cnt = (long)P >= kSortSplitMinPairs ? take((size_t)kSortMaxGroups * (size_t)n_experts * 4) : 0;
  L.xhi = take((size_t)T * Hp);
  L.xlo = take((size_t)T * Hp);
  L.xshi = take((size_t)T * Hp / kBlock);
  L.xslo = take((size_t)T * Hp / kBlock);
  L.hhi = take(P * Ip);
  L.hlo = take(P * Ip);
  L.hshi = take(P * Ip / kBlock);
  L.hslo = take(P * Ip / kBlock);
  L.ypair = take(P * (size_t)hidden * 4);
  L.bytes = off;
  L.nb_max = nb_max;
  L.Hp = (int)Hp;
  L.Ip = (int)Ip;
  return L;
}

template <int TERMS, bool NT>
static hipError_t batched_ffn(const uint16_t* x, const int32_t* ids, const float* w, int T, int k,
                              const uint8_t* packed, int n_experts, int hidden, int inter,
                              uint16_t* y, void* workspace, hipStream_t s) {
  const BatchedLayout B = batched_layout(T, k, n_experts, hidden, inter);
  const PackedLayout L = packed_layout(hidden, inter);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + B.offsets);
  int32_t* perm = reinterpret_cast<int32_t*>(ws + B.perm);
  int32_t* bexp = reinterpret_cast<int32_t*>(ws + B.blk_expert);
  int32_t* brow0 = reinterpret_cast<int32_t*>(ws + B.blk_row0);
  int32_t* nblk = reinterpret_cast<int32_t*>(ws + B.n_blocks);
  const long P = (long)T * k;
  if (P > 0x7fffffffL) return hipErrorInvalidValue;

  hipError_t e;
  if (P < kSortSplitMinPairs) {
    const uint32_t sort_lds = (uint32_t)((3 * n_experts + kSortThreads) * sizeof(int));
    e = launch_kernel(kKindBatchedSort, sort_kernel, dim3(1), dim3(kSortThreads), sort_lds, s, ids,
                      (int)P, n_experts, offsets, perm, bexp, brow0, nblk);
    if (e != hipSuccess) return e;
  } else {  // many workgroups, each over `chunk` consecutive pairs
    const int G = (int)std::min<long>(kSortMaxGroups, (P + 1023) / 1024);
    const int chunk = (int)((P + G - 1) / G);
    int32_t* cnt = reinterpret_cast<int32_t*>(ws + B.sort_cnt);
    const uint32_t hist_lds = (uint32_t)(n_experts * sizeof(int));
    e = launch_kernel(kKindBatchedSort, sort_count_kernel, dim3(G), dim3(kSortWGThreads), hist_lds, s,
                      ids, (int)P, n_experts, chunk, cnt);
    if (e != hipSuccess) return e;
    const uint32_t scan_lds = (uint32_t)((n_experts + kSortThreads) * sizeof(int));
    e = launch_kernel(kKindBatchedSort, sort_scan_kernel, dim3(1), dim3(kSortThreads), scan_lds, s, G,
                      n_experts, cnt, offsets, bexp, brow0, nblk);
    if (e != hipSuccess) return e;
    e = launch_kernel(kKindBatchedSort, sort_scatter_kernel, dim3(G), dim3(kSortWGThreads), hist_lds,
                      s, ids, (int)P, n_experts, chunk, cnt, perm);
    if (e != hipSuccess) return e;
  }

  const long qn = (long)T * (B.Hp / kBlock);
  e = launch_kernel(kKindBatchedQuant, quant_x_kernel<TERMS>, dim3((unsigned)((qn + 255) / 256)), dim3(256), 0,
                    s, x, T, hidden, B.Hp, ws + B.xhi, ws + B.xlo, ws + B.xshi, ws + B.xslo);
  if (e != hipSuccess) return e;

  const int gu_tiles = (inter + kBN - 1) / kBN;
  static_assert(kXcds == 8, "grid rounding below");
  const long gu_grid = ((long)B.nb_max * gu_tiles + 7) / 8 * 8;  // a multiple of the XCD count
  if (gu_grid > 0x7fffffffL) return hipErrorInvalidValue;
  e = launch_kernel(kKindBatchedGateUp, gemm_gate_up_kernel<TERMS, NT>, dim3((unsigned)gu_grid), dim3(kBThreads), 0,
                    s, ws + B.xhi, ws + B.xlo, ws + B.xshi, ws + B.xslo, B.Hp, perm, bexp, brow0,
                    offsets, nblk, k, packed, L.stride, L.m[0].codes, L.m[1].codes, L.m[0].scales,
                    L.m[1].scales, hidden, inter, gu_tiles, ws + B.hhi, ws + B.hlo, ws + B.hshi,
                    ws + B.hslo, B.Ip);
  if (e != hipSuccess) return e;

  const int dn_tiles = (hidden + kBND - 1) / kBND;
  const long dn_grid = ((long)B.nb_max * dn_tiles + 7) / 8 * 8;
  if (dn_grid > 0x7fffffffL) return hipErrorInvalidValue;
  float* ypair = reinterpret_cast<float*>(ws + B.ypair);
  e = launch_kernel(kKindBatchedDown, gemm_down_kernel<TERMS, NT>, dim3((unsigned)dn_grid), dim3(kBThreads), 0, s,
                    ws + B.hhi, ws + B.hlo, ws + B.hshi, ws + B.hslo, B.Ip, perm, w, bexp, brow0,
                    offsets, nblk, packed, L.stride, L.m[2].codes, L.m[2].scales, hidden, inter,
                    dn_tiles, ypair);
  if (e != hipSuccess) return e;

  return launch_combine_pairs(ids, w, T, k, n_experts, hidden, ypair, y, s);
}

hipError_t launch_batched_ffn(const uint16_t* x, const int32_t* ids, const float* w, int T, int k,
                              const uint8_t* packed, int n_experts, int hidden, int inter,
                              uint16_t* y, void* workspace, int terms, hipStream_t s) {
  // non-temporal weight loads unless the experts average a full M-block of pairs or more
  const bool nt = (long)T * k < (long)kBlockRows * n_experts;
#define MOE_FP4_BATCHED(TM, N) \
  batched_ffn<TM, N>(x, ids, w, T, k, packed, n_experts, hidden, inter, y, workspace, s)
  if (terms == 1) return nt ? MOE_FP4_BATCHED(1, true) : MOE_FP4_BATCHED(1, false);
  if (terms == 2) return nt ? MOE_FP4_BATCHED(2, true) : MOE_FP4_BATCHED(2, false);
#undef MOE_FP4_BATCHED
  return hipErrorInvalidValue;
}

hipError_t launch_combine_pairs(const int32_t* ids, const float* w, int T, int k, int n_experts,
                                int hidden, const float* ypair, uint16_t* y, hipStream_t s) {
  const int col_blocks = (hidden + kCombineCols - 1) / kCombineCols;
  const long grid = (long)T * col_blocks;
  if (grid > 0x7fffffffL) return hipErrorInvalidValue;
  return launch_kernel(kKindBatchedCombine, combine_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                       ids, w, k, n_experts, hidden, col_blocks, ypair, y);
}

size_t debug_act_quant_bytes(int T, int H) {
  const size_t Hp = (size_t)(H + 127) / 128 * 128;
  return 2 * (size_t)T * Hp + 2 * (size_t)T * (Hp / kBlock);
}

hipError_t launch_debug_act_quant(const uint16_t* x, int T, int H, int terms, void* ws, float* out,
                                  hipStream_t s) {
  if ((long)T * H > 0x7fffffffL * 256L) return hipErrorInvalidValue;
  uint8_t* w = static_cast<uint8_t*>(ws);
  if (terms == 1) return debug_act_quant<1>(x, T, H, w, out, s);
  if (terms == 2) return debug_act_quant<2>(x, T, H, w, out, s);
  return hipErrorInvalidValue;
}

}  // namespace moe_fp4
