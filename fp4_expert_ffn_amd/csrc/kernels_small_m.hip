// Small-M routed-expert FFN: a few tokens per call (several draft tokens of one sequence, a
// few streams). The (token, slot) pairs that chose one expert read its weights once for all
// of them: each expert's stream feeds up to MR matrix-core rows, one per member pair, in the
// same weight-streaming scheme as the one-pair decode kernels ([A100-FP4], section
// 批处理不是「同时处理几个人」: batching pays only where several tokens share the weights
// read; [8GB-GPU], section 每 token 字节数决定一切: the bytes streamed per token set the time).
#include <algorithm>

#include "moe_fp4_device.hpp"
#include "moe_fp4_gemv.hpp"
#include "moe_fp4_internal.hpp"

namespace moe_fp4 {

namespace {

// ---------------------------------------------------------------------------------------
// Small-M path: a few tokens per call (several draft tokens of one sequence, a few
// streams), where tokens often choose the same experts. The (token, slot) pairs that chose
// one expert share its weight stream: in ascending pair index they form groups of up to MR
// members; the workgroups of a group's first member compute every member (matrix-core rows
// 0..m-1 are the members' tokens) and the other members' workgroups exit at once. Rows of
// the matrix-core product are independent and each row's arithmetic is the decode kernels',
// so gate/up's h equals the decode path's bit for bit; down writes each pair's weighted
// fp32 row and the fixed-order combine of the grouped path sums a token's rows.
//
// The members' activation rows are staged in LDS, at most kSmallLdsBytes per workgroup so
// that as many workgroups fit on a compute unit as the decode kernels' register budget
// allows. Word w of row r sits at r * nw + (w ^ (r & 3)): the lanes of different rows that
// read the same word of their rows meet different banks. Lanes of matrix-core rows >= m
// read row m - 1 (their results are never stored); K-tail lanes read their row's first
// chunk against zero weights. After the products the same LDS holds the waves' partial
// sums for the cross-wave reduction.
// ---------------------------------------------------------------------------------------
constexpr int kSmallMaxPairs = 256;       // T * k scanned for the grouping (four ballots)
constexpr int kSmallLdsBytes = 32768;     // staged rows per workgroup
constexpr int kSmallStage = kSmallLdsBytes / (16 * kGUThreads);  // 16-byte words per thread
static_assert(kGUThreads == kTile * kTile, "one (member, column) per thread in the epilogues");

// The grouping, evaluated by every wave from the ids alone (all values wave-uniform): the
// pairs that chose e = ids[pair] are numbered in pair order; `pair` leads a group when its
// number is a multiple of MR, and the group is it and the next up to MR - 1 pairs of e.
// Returns the member count m (0 for a non-leader or an invalid id), the members in bytes
// 0..m-1 of *rows (ascending pair indices, each below kSmallMaxPairs) and the expert in *e_out.
template <int MR>
__device__ __forceinline__ int small_group(const int32_t* __restrict__ ids, int P, int pair,
                                           int n_experts, int lane, uint64_t* rows, int* e_out) {
  static_assert(MR <= 8 && kSmallMaxPairs <= 256, "members packed as bytes of one 64-bit word");
  const int e = ids[pair];
  const bool valid = e >= 0 && e < n_experts;
  unsigned long long mk[kSmallMaxPairs / 64];
#pragma unroll
  for (int i = 0; i < kSmallMaxPairs / 64; ++i) {
    const int q = lane + 64 * i;
    const int eq = ids[min(q, P - 1)];
    mk[i] = __ballot(valid && q < P && eq == e);  // every lane votes
  }
  *e_out = e;
  *rows = 0;
  if (!valid) return 0;
  int rank = 0;
#pragma unroll
  for (int i = 0; i < kSmallMaxPairs / 64; ++i) {
    const int lo = 64 * i;
    if (pair >= lo + 64) {
      rank += __popcll(mk[i]);
      mk[i] = 0ull;
    } else if (pair > lo) {
      const unsigned long long below = (1ull << (pair - lo)) - 1ull;
      rank += __popcll(mk[i] & below);
      mk[i] &= ~below;
    }
  }
  if (rank % MR != 0) return 0;
  int m = 0;
  uint64_t packed_rows = 0;
#pragma unroll
  for (int s = 0; s < MR; ++s) {
    int at = -1;
#pragma unroll
    for (int i = kSmallMaxPairs / 64 - 1; i >= 0; --i)
      if (mk[i] != 0ull) at = i;
    if (at >= 0) {
      unsigned long long b = mk[0];
#pragma unroll
      for (int i = 1; i < kSmallMaxPairs / 64; ++i)
        if (at == i) b = mk[i];
      const int bit = __ffsll((long long)b) - 1;
      packed_rows |= (uint64_t)(64 * at + bit) << (8 * s);
#pragma unroll
      for (int i = 0; i < kSmallMaxPairs / 64; ++i)
        if (at == i) mk[i] &= mk[i] - 1ull;
      m = s + 1;
    }
  }
  *rows = packed_rows;
  return m;
}

__device__ __forceinline__ int pick_row(uint64_t rows, int r) { return (int)((rows >> (8 * r)) & 255u); }

// The members' rows straight from global memory into LDS (global_load_lds_dwordx4: lane L
// of a wave writes 16 bytes at the wave's LDS base + 16 L, no registers involved). Round
// u of wave wv fills the 64 slots from (u * kGUWaves + wv) * 64 of the swizzled [m x nw]
// block; each lane loads the source word its slot holds (row rows[r] / div: the token for
// gate/up, the pair for down). Lanes past the block stay idle.
__device__ __forceinline__ void stage_rows(const uint4* src, uint64_t rows, int div, int m, int nw,
                                           int wv, int lane, uint4* smem_wave_base) {
  const int total = m * nw;
#pragma unroll
  for (int u = 0; u < kSmallStage; ++u) {
    const int blk = (u * kGUWaves + wv) * 64;
    const int p = blk + lane;
    if (p < total) {
      const int r = p / nw, ws = p - r * nw;
      __builtin_amdgcn_global_load_lds(src + (size_t)(pick_row(rows, r) / div) * nw + (ws ^ (r & 3)),
                                       smem_wave_base + u * kGUWaves * 64, 16, 0, 0);
    }
  }
}

// Byte offsets in LDS of the A operand words ms = 0..3 of this lane for chunk 0; a K-tail
// lane adds 0 - 64 g instead of 256 c, which gives words 0..3 of its row.
__device__ __forceinline__ void stage_a_offsets(int j, int g, int m, int nw, uint32_t (&a)[4]) {
  const int rj = min(j, m - 1);
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) a[ms] = (uint32_t)(rj * nw + 4 * g + (ms ^ (rj & 3))) * 16u;
}

// Gate/up for a group (tile of 16 rows of gate and up; the waves split K as in gate_up_kernel).
template <int MR>
__global__ __launch_bounds__(kGUThreads) __attribute__((amdgpu_waves_per_eu(MOE_FP4_GU_MIN_WAVES)))
void gate_up_multi_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ ids, int k,
                          int P, const uint8_t* packed, size_t stride, size_t off_gc,
                          size_t off_uc, size_t off_gs, size_t off_us, int n_experts, int H, int I,
                          int tiles_per_pair, uint16_t* __restrict__ hbuf) {
  extern __shared__ uint4 smem[];
  const int pair = blockIdx.x / tiles_per_pair;
  const int row0 = (blockIdx.x - pair * tiles_per_pair) * kTile;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int KB = H / kBlock;
  const int nch = (KB + 3) / 4;
  const int nx = H / 8;

  uint64_t rows;
  int e;
  const int m = small_group<MR>(ids, P, pair, n_experts, lane, &rows, &e);
  if (m == 0) return;  // the same in every wave

  // 1. the members' x rows into LDS
  stage_rows(reinterpret_cast<const uint4*>(x), rows, k, m, nx, wv, lane, smem + wv * 64);

  // 2. this wave's first batch of weights (as in gate_up_kernel)
  const int c_begin = wv * nch / kGUWaves;
  const int c_end = (wv + 1) * nch / kGUWaves;
  const size_t tbase = (size_t)(row0 / kTile) * kTile * KB;
  const uint8_t* base = packed + (size_t)e * stride;
  const uint4* gcodes = reinterpret_cast<const uint4*>(base + off_gc) + tbase;
  const uint4* ucodes = reinterpret_cast<const uint4*>(base + off_uc) + tbase;
  const uint8_t* gscales = base + off_gs + tbase;
  const uint8_t* uscales = base + off_us + tbase;
  uint4 cg[kGUBatch], cu[kGUBatch];
  uint32_t sg[kGUBatch], su[kGUBatch];
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int q = 0; q < kGUBatch; ++q) {
      const int c = max(min(c0 + q, c_end - 1), 0);
      const int w = (4 * c + g < KB) ? 64 * c + lane : 64 * c;
      cg[q] = ld_stream(gcodes + w);
      cu[q] = ld_stream(ucodes + w);
      sg[q] = ld_scale(gscales + w);
      su[q] = ld_scale(uscales + w);
    }
  };
  load_batch(c_begin);  // unconditional (a wave without chunks loads chunk 0, unused)
  __syncthreads();

  const char* lds = reinterpret_cast<const char*>(smem);
  uint32_t a_off[4];
  stage_a_offsets(j, g, m, nx, a_off);
  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  auto mfma_chunk = [&](uint32_t cb, const uint4& wg, const uint4& wu, float fg, float fu) {
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
      const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(lds + a_off[ms] + cb));
      accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, fp4x8_to_bf16(dword(wg, ms), fg), accg, 0, 0, 0);
      accu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, fp4x8_to_bf16(dword(wu, ms), fu), accu, 0, 0, 0);
    }
  };
  for (int c0 = c_begin; c0 < c_end; c0 += kGUBatch) {
    if (c0 + kGUBatch <= c_end && 4 * (c0 + kGUBatch) <= KB) {
#pragma unroll
      for (int q = 0; q < kGUBatch; ++q)
        mfma_chunk((uint32_t)(c0 + q) * 256u, cg[q], cu[q], scale_operand(sg[q]),
                   scale_operand(su[q]));
    } else {
#pragma unroll
      for (int q = 0; q < kGUBatch; ++q) {
        const int c = c0 + q;
        const bool bv = (c < c_end) && (4 * c + g < KB);
        mfma_chunk(bv ? (uint32_t)c * 256u : 0u - 64u * (uint32_t)g, bv ? cg[q] : make_uint4(0, 0, 0, 0),
                   bv ? cu[q] : make_uint4(0, 0, 0, 0), scale_operand(bv ? sg[q] : 127u),
                   scale_operand(bv ? su[q] : 127u));
      }
    }
    if (c0 + kGUBatch < c_end) load_batch(c0 + kGUBatch);
  }
  // partial sums over LDS: [wave][member][column], gate then up; accumulator element q of
  // this lane is row 4 (lane / 16) + q, column lane % 16
  __syncthreads();
  float* red_g = reinterpret_cast<float*>(smem);
  float* red_u = red_g + kGUWaves * MR * kTile;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 4 * g + q;
    if (r < m) {
      red_g[(wv * MR + r) * kTile + j] = accg[q];
      red_u[(wv * MR + r) * kTile + j] = accu[q];
    }
  }
  __syncthreads();
  {
    const int r = tid / kTile, c = tid % kTile;  // one (member, column) per thread
    if (r < m && row0 + c < I) {
      float gs = 0.f, us = 0.f;
#pragma unroll
      for (int w = 0; w < kGUWaves; ++w) {
        gs += red_g[(w * MR + r) * kTile + c];
        us += red_u[(w * MR + r) * kTile + c];
      }
      hbuf[(size_t)pick_row(rows, r) * I + row0 + c] = f32_to_bf16_rne(silu_f32(gs) * us);
    }
  }
}

// Down for a group: each member's y_e row times its router weight, fp32, into ypair.
template <int MR>
__global__ __launch_bounds__(kGUThreads) __attribute__((amdgpu_waves_per_eu(MOE_FP4_GU_MIN_WAVES)))
void down_multi_kernel(const int32_t* __restrict__ ids, const float* __restrict__ wts, int P,
                       const uint8_t* packed, size_t stride, size_t off_dc,
                       size_t off_ds, int n_experts, int H, int I, int tiles_per_pair,
                       const uint16_t* __restrict__ hbuf, float* __restrict__ ypair) {
  extern __shared__ uint4 smem[];
  const int pair = blockIdx.x / tiles_per_pair;
  const int row0 = (blockIdx.x - pair * tiles_per_pair) * kTile;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int KB = I / kBlock;
  const int nch = (KB + 3) / 4;
  const int nh = I / 8;

  uint64_t rows;
  int e;
  const int m = small_group<MR>(ids, P, pair, n_experts, lane, &rows, &e);
  if (m == 0) return;

  stage_rows(reinterpret_cast<const uint4*>(hbuf), rows, 1, m, nh, wv, lane, smem + wv * 64);

  const int c_begin = wv * nch / kGUWaves;
  const int c_end = (wv + 1) * nch / kGUWaves;
  const size_t tbase = (size_t)(row0 / kTile) * kTile * KB;
  const uint8_t* base = packed + (size_t)e * stride;
  const uint4* dcodes = reinterpret_cast<const uint4*>(base + off_dc) + tbase;
  const uint8_t* dscales = base + off_ds + tbase;
  uint4 cd[kGUBatch];
  uint32_t sd[kGUBatch];
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int q = 0; q < kGUBatch; ++q) {
      const int c = max(min(c0 + q, c_end - 1), 0);
      const int w = (4 * c + g < KB) ? 64 * c + lane : 64 * c;
      cd[q] = ld_stream(dcodes + w);
      sd[q] = ld_scale(dscales + w);
    }
  };
  load_batch(c_begin);  // unconditional (a wave without chunks loads chunk 0, unused)
  __syncthreads();

  const char* lds = reinterpret_cast<const char*>(smem);
  uint32_t a_off[4];
  stage_a_offsets(j, g, m, nh, a_off);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  auto mfma_chunk = [&](uint32_t cb, const uint4& wd, float fd) {
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
      const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(lds + a_off[ms] + cb));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, fp4x8_to_bf16(dword(wd, ms), fd), acc, 0, 0, 0);
    }
  };
  for (int c0 = c_begin; c0 < c_end; c0 += kGUBatch) {
    if (c0 + kGUBatch <= c_end && 4 * (c0 + kGUBatch) <= KB) {
#pragma unroll
      for (int q = 0; q < kGUBatch; ++q)
        mfma_chunk((uint32_t)(c0 + q) * 256u, cd[q], scale_operand(sd[q]));
    } else {
#pragma unroll
      for (int q = 0; q < kGUBatch; ++q) {
        const int c = c0 + q;
        const bool bv = (c < c_end) && (4 * c + g < KB);
        mfma_chunk(bv ? (uint32_t)c * 256u : 0u - 64u * (uint32_t)g, bv ? cd[q] : make_uint4(0, 0, 0, 0),
                   scale_operand(bv ? sd[q] : 127u));
      }
    }
    if (c0 + kGUBatch < c_end) load_batch(c0 + kGUBatch);
  }
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 4 * g + q;
    if (r < m) red[(wv * MR + r) * kTile + j] = acc[q];
  }
  __syncthreads();
  {
    const int r = tid / kTile, c = tid % kTile;
    if (r < m && row0 + c < H) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kGUWaves; ++w) sum += red[(w * MR + r) * kTile + c];
      const int pr = pick_row(rows, r);
      ypair[(size_t)pr * H + row0 + c] = wts[pr] * sum;
    }
  }
}

}  // namespace

// Rows per group for T tokens: the largest power of two <= min(T, 8) whose staged rows
// (bf16, max(hidden, inter) wide) fit in kSmallLdsBytes; 1 means the path does not apply.
int small_m_rows(int T, int hidden, int inter) {
  const size_t row = (size_t)std::max(hidden, inter) * 2;
  int mr = 8;
  while (mr > 1 && (mr > T || (size_t)mr * row > (size_t)kSmallLdsBytes)) mr /= 2;
  return mr;
}

size_t small_m_workspace_bytes(int T, int k, int hidden, int inter) {
  const size_t P = (size_t)T * (size_t)k;
  return align_up256(P * (size_t)inter * 2) + align_up256(P * (size_t)hidden * 4);
}

template <int MR>
hipError_t small_m_launch(const uint16_t* x, const int32_t* ids, const float* w, int T, int k,
                          const uint8_t* packed, int n_experts, int H, int I, void* workspace,
                          uint16_t* y, hipStream_t s) {
  const PackedLayout L = packed_layout(H, I);
  const int P = T * k;
  uint16_t* hbuf = static_cast<uint16_t*>(workspace);
  float* ypair = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                          align_up256((size_t)P * (size_t)I * 2));
  const int gu_tiles = (I + kTile - 1) / kTile;
  const int dn_tiles = H / kTile;
  // staged rows, or the partial sums (gate and up) if larger
  const uint32_t lds_gu = (uint32_t)std::max(MR * (H / 8) * 16, 2 * kGUWaves * MR * kTile * 4);
  const uint32_t lds_dn = (uint32_t)std::max(MR * (I / 8) * 16, kGUWaves * MR * kTile * 4);
  if (lds_gu > (uint32_t)kSmallLdsBytes || lds_dn > (uint32_t)kSmallLdsBytes)
    return hipErrorInvalidValue;
  hipError_t e = launch_kernel(kKindSmallGateUp, gate_up_multi_kernel<MR>,
                               dim3((unsigned)((long)P * gu_tiles)), dim3(kGUThreads), lds_gu, s, x,
                               ids, k, P, packed, L.stride, L.m[0].codes, L.m[1].codes,
                               L.m[0].scales, L.m[1].scales, n_experts, H, I, gu_tiles, hbuf);
  if (e != hipSuccess) return e;
  e = launch_kernel(kKindSmallDown, down_multi_kernel<MR>, dim3((unsigned)((long)P * dn_tiles)),
                    dim3(kGUThreads), lds_dn, s, ids, w, P, packed, L.stride, L.m[2].codes,
                    L.m[2].scales, n_experts, H, I, dn_tiles, (const uint16_t*)hbuf, ypair);
  if (e != hipSuccess) return e;
  return launch_combine_pairs(ids, w, T, k, n_experts, H, ypair, y, s);
}

hipError_t launch_small_m_ffn(const uint16_t* x, const int32_t* ids, const float* w, int T, int k,
                              const uint8_t* packed, int n_experts, int hidden, int inter,
                              void* workspace, uint16_t* y, hipStream_t s) {
  if ((long)T * k > kSmallMaxPairs) return hipErrorInvalidValue;
  switch (small_m_rows(T, hidden, inter)) {
    case 8: return small_m_launch<8>(x, ids, w, T, k, packed, n_experts, hidden, inter, workspace, y, s);
    case 4: return small_m_launch<4>(x, ids, w, T, k, packed, n_experts, hidden, inter, workspace, y, s);
    case 2: return small_m_launch<2>(x, ids, w, T, k, packed, n_experts, hidden, inter, workspace, y, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe_fp4
