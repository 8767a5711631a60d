// Routed expert FFN, one (token, slot) pair at a time, on the bf16 matrix cores.
//
// Stage 1 (gate_up): g = W_gate[e] x, u = W_up[e] x, h = silu(g) * u for every pair
//   (t, j) with a valid id; h goes to the workspace as bf16, natural order [pair][I].
// Stage 2 (down_combine): y[t, n] = sum over the token's valid slots, in canonical order
//   (ascending expert id), of w_j * (W_down[e_j] h_j)[n]; y is written as bf16.
//
// Both stages are matrix-vector products with FP4 weights. A workgroup owns a tile of 16
// weight rows; its wavefronts split K. Per 128-element chunk of K, lane l (column
// j = l % 16 of the MFMA, group g = l / 16) loads the 16 bytes of one 32-code block of
// weight row (row0 + j), block 4 * chunk + g: a wavefront load covers 16 rows x 4 blocks.
// The block is dequantised in registers by the hardware FP4 -> bf16 conversion, its ue8m0
// scale applied in the same instruction (exact for every scale byte; see scale_operand), and fed as the B
// operand of v_mfma_f32_16x16x32_bf16; the token's activations are row 0 of the A operand
// (read from LDS by the four lanes with l % 16 == 0, zeros elsewhere), so row 0 of the
// 16 x 16 accumulator holds the 16 dot products. The weights are never expanded in memory:
// storage and compute formats meet only in registers ([A100-FP4], section
// 「FP4非対応」という言葉を疑う). The same lane order is used for the A and B K-slots, so
// each MFMA covers elements 32g + 8m .. 32g + 8m + 7 of the chunk for m = 0..3.
#include <algorithm>

#include "moe_fp4_device.hpp"
#include "moe_fp4_gemv.hpp"
#include "moe_fp4_internal.hpp"

namespace moe_fp4 {

namespace {

// Down/combine launch shape, tuned by measurement on MI355X; overridable at build time.
#ifndef MOE_FP4_DC_WAVES
#define MOE_FP4_DC_WAVES 16     // wavefronts per down/combine tile
#endif
#ifndef MOE_FP4_DC_BATCH
#define MOE_FP4_DC_BATCH 3      // (expert, chunk) steps loaded per wave before use
#endif

constexpr int kDCWaves = MOE_FP4_DC_WAVES;
constexpr int kDCThreads = kDCWaves * 64;
constexpr int kDCBatch = MOE_FP4_DC_BATCH;
// the down kernel stages a token's h vectors (at most kMaxLdsH bytes) in at most four
// 16-byte words per thread
static_assert(4 * kDCThreads * 16 >= 65536, "MOE_FP4_DC_WAVES must be at least 16");

// ---------------------------------------------------------------------------------------
// Stage 1: gate/up/SiLU. Workgroup = one tile of 16 rows of gate and up of one pair; the
// kGUWaves waves take equal shares of the K chunks, in batches of kGUBatch chunks.
// LDS: the token's x (H bf16) followed by four zero 16-byte words.
// ---------------------------------------------------------------------------------------
// The kernel is kept to MOE_FP4_GU_MIN_WAVES wavefronts per SIMD so that one launch's
// tiles are resident together (no second round at the end).
template <int XR>
__global__ __launch_bounds__(kGUThreads) __attribute__((amdgpu_waves_per_eu(MOE_FP4_GU_MIN_WAVES)))
void gate_up_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ ids, int k,
                    const uint8_t* __restrict__ packed, size_t stride, size_t off_gc,
                    size_t off_uc, size_t off_gs, size_t off_us, int n_experts, int H, int I,
                    int tiles_per_pair, uint16_t* __restrict__ hbuf) {
  extern __shared__ uint4 smem[];
  __shared__ float red_g[kGUWaves][kTile], red_u[kGUWaves][kTile];
  const int tile = blockIdx.x;
  const int pair = tile / tiles_per_pair;
  const int row0 = (tile - pair * tiles_per_pair) * kTile;
  const int t = pair / k;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int KB = H / kBlock;
  const int nch = (KB + 3) / 4;  // 128-element chunks of K
  const int nx = H / 8;          // 16-byte words of x

  // 1. x into registers (XR rounds of the workgroup cover H; indices clamped, so every
  // load is issued). x does not depend on the expert, so it goes first.
  constexpr int kXRounds = XR;
  uint4 xr[kXRounds];
  const uint4* xv = reinterpret_cast<const uint4*>(x + (size_t)t * H);
#pragma unroll
  for (int r = 0; r < kXRounds; ++r) {
    xr[r] = make_uint4(0, 0, 0, 0);
    if (r * kGUThreads < nx) xr[r] = xv[min(tid + r * kGUThreads, nx - 1)];
  }

  const int e = ids[pair];
  if (e < 0 || e >= n_experts) return;  // whole workgroup

  // 2. this wave's first batch of weights
  const int c_begin = wv * nch / kGUWaves;
  const int c_end = (wv + 1) * nch / kGUWaves;
  // tile-major packed layout: word (tile, c, g, j) at tile * 16 * KB + 64 c + lane
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
      const int c = min(c0 + q, c_end - 1);
      const int w = (4 * c + g < KB) ? 64 * c + lane : 64 * c;  // blocks past K: any valid word
      cg[q] = ld_stream(gcodes + w);
      cu[q] = ld_stream(ucodes + w);
      sg[q] = ld_scale(gscales + w);
      su[q] = ld_scale(uscales + w);
    }
  };
  if (c_begin < c_end) load_batch(c_begin);

  // 3. x into LDS
#pragma unroll
  for (int r = 0; r < kXRounds; ++r) {
    const int i = tid + r * kGUThreads;
    if (r * kGUThreads < nx && i < nx) smem[i] = xr[r];
  }
  if (tid < 4) smem[nx + tid] = make_uint4(0, 0, 0, 0);
  __syncthreads();

  // A operand from LDS: the lanes of row 0 (j == 0) read x words 16 c + 4 g + m, the other
  // lanes the 4-word zero area; byte addresses, the 16 m offset folded into the reads.
  const char* lds = reinterpret_cast<const char*>(smem);
  const uint32_t zero_addr = (uint32_t)nx * 16u;
  const uint32_t a_lane = (j == 0) ? (uint32_t)(64 * g) : zero_addr;
  const uint32_t a_step = (j == 0) ? 256u : 0u;
  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  auto mfma_chunk = [&](uint32_t a_addr, const uint4& wg, const uint4& wu, float fg, float fu) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(lds + a_addr + 16 * m));
      accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, fp4x8_to_bf16(dword(wg, m), fg), accg, 0, 0, 0);
      accu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, fp4x8_to_bf16(dword(wu, m), fu), accu, 0, 0, 0);
    }
  };
  for (int c0 = c_begin; c0 < c_end; c0 += kGUBatch) {
    if (c0 + kGUBatch <= c_end && 4 * (c0 + kGUBatch) <= KB) {  // wave-uniform: all blocks exist
#pragma unroll
      for (int q = 0; q < kGUBatch; ++q)
        mfma_chunk(a_lane + (uint32_t)(c0 + q) * a_step, cg[q], cu[q], scale_operand(sg[q]),
                   scale_operand(su[q]));
    } else {
#pragma unroll
      for (int q = 0; q < kGUBatch; ++q) {
        const int c = c0 + q;
        const bool bv = (c < c_end) && (4 * c + g < KB);  // wave-uniform c, per-lane block
        mfma_chunk(bv ? a_lane + (uint32_t)c * a_step : zero_addr,
                   bv ? cg[q] : make_uint4(0, 0, 0, 0), bv ? cu[q] : make_uint4(0, 0, 0, 0),
                   scale_operand(bv ? sg[q] : 127u), scale_operand(bv ? su[q] : 127u));
      }
    }
    if (c0 + kGUBatch < c_end) load_batch(c0 + kGUBatch);
  }
  // row 0 of the accumulators: lanes 0..15, element 0
  if (lane < kTile) {
    red_g[wv][lane] = accg[0];
    red_u[wv][lane] = accu[0];
  }
  __syncthreads();
  if (tid < kTile && row0 + tid < I) {
    float gs = 0.f, us = 0.f;
#pragma unroll
    for (int w = 0; w < kGUWaves; ++w) {
      gs += red_g[w][tid];
      us += red_u[w][tid];
    }
    hbuf[(size_t)pair * I + row0 + tid] = f32_to_bf16_rne(silu_f32(gs) * us);
  }
}

// ---------------------------------------------------------------------------------------
// Stage 2: down projection and weighted combine. Workgroup = one tile of 16 output rows of
// one token. The token's valid slots are put in canonical order (ascending expert id, then
// weight bits, then slot; invalid ids dropped) and the (slot, chunk) steps are split evenly
// over the kDCWaves waves; each wave keeps one accumulator for the slot it is on and
// stores it to LDS when it moves on. The final sum over waves and slots runs in a fixed
// order, so permuting a token's (id, weight) pairs gives bit-identical output.
// Load order per thread: wave 0 first loads the token's ids and weights; every thread then
// loads its share of the token's k h vectors (natural slot order, so the addresses need no
// routing data), then its first batch of down weights, then does the LDS stores. Every
// load is issued (indices clamped to valid data) and every store is unconditional (surplus
// words go to a dummy LDS word), so the stores wait for the h loads only. Per-slot expert bases and slot numbers sit in one VGPR per lane and
// are read with readlane at the wave-uniform slot index.
// LDS: h of the KT slots (bf16, natural order) then four zero 16-byte words and a dummy.
// ---------------------------------------------------------------------------------------
template <int KT, int HR>
__global__ __launch_bounds__(kDCThreads) void down_combine_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ wts, int T,
    const uint8_t* __restrict__ packed, size_t stride, size_t off_dc, size_t off_ds,
    int n_experts, int H, int I, int tiles_per_token, const uint16_t* __restrict__ hbuf,
    uint16_t* __restrict__ y) {
  extern __shared__ uint4 smem[];
  __shared__ float red[kDCWaves][KT][kTile];
  __shared__ int s_sid[KT], s_slot[KT], s_nv;
  __shared__ float s_w[KT];
  const int t = blockIdx.x / tiles_per_token;
  const int row0 = (blockIdx.x - t * tiles_per_token) * kTile;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int j16 = lane & 15;
  const int g = lane >> 4;
  const int KBI = I / kBlock;
  const int nch = (KBI + 3) / 4;
  const int hx = I / 8;      // 16-byte words per h vector
  const int hw = KT * hx;    // 16-byte words of the token's k h vectors

  // 1. wave 0: the token's ids and weights (clamped, unconditional loads) go out first, so
  // the slot table below does not wait behind the h vectors (loads return in order)
  int ej_raw = 0;
  uint32_t wj_raw = 0u;
  if (tid < 64) {  // wave-uniform
    const int jc = min(tid, KT - 1);
    ej_raw = ids[(size_t)t * KT + jc];
    wj_raw = __float_as_uint(wts[(size_t)t * KT + jc]);
  }

  // 2. the token's h vectors into registers (named registers: an array live across the
  // table code below would be placed in private memory)
  const uint4* hv = reinterpret_cast<const uint4*>(hbuf + (size_t)t * KT * I);
  static_assert(HR >= 1 && HR <= 4, "h rounds");
  uint4 hr0 = hv[min(tid, hw - 1)], hr1 = hr0, hr2 = hr0, hr3 = hr0;
  if constexpr (HR > 1) hr1 = hv[min(tid + kDCThreads, hw - 1)];
  if constexpr (HR > 2) hr2 = hv[min(tid + 2 * kDCThreads, hw - 1)];
  if constexpr (HR > 3) hr3 = hv[min(tid + 3 * kDCThreads, hw - 1)];

  // 3. canonical slot order: lane jj < KT of wave 0 ranks slot jj; lane 0 writes the table
  // in rank order, entries past the valid slots pointing at expert 0 / slot 0 (used only
  // by clamped loads whose results are discarded)
  if (tid < 64) {
    const int jj = tid;
    const int ej = (jj < KT) ? ej_raw : -1;
    const uint32_t wj = (jj < KT) ? wj_raw : 0u;
    const bool okj = jj < KT && ej >= 0 && ej < n_experts;
    int rank = 0;
#pragma unroll
    for (int i = 0; i < KT; ++i) {  // readlane: a register read, not an LDS round trip
      const int ei = __builtin_amdgcn_readlane(ej, i);
      const uint32_t wi = (uint32_t)__builtin_amdgcn_readlane((int)wj, i);
      const bool oki = ei >= 0 && ei < n_experts;
      const bool before = ei < ej || (ei == ej && (wi < wj || (wi == wj && i < jj)));
      rank += (oki && before) ? 1 : 0;
    }
    const int nvl = __popcll(__ballot(okj));
#pragma unroll
    for (int r = 0; r < KT; ++r) {
      const int sr = __ffsll((long long)__ballot(okj && rank == r)) - 1;  // wave-uniform
      const int src = sr < 0 ? 0 : sr;
      const int er = __builtin_amdgcn_readlane(ej, src);
      const uint32_t wr = (uint32_t)__builtin_amdgcn_readlane((int)wj, src);
      if (lane == 0) {
        s_sid[r] = sr < 0 ? 0 : er;
        s_slot[r] = src;
        s_w[r] = sr < 0 ? 0.f : __uint_as_float(wr);
      }
    }
    if (lane == 0) s_nv = nvl;
  }
  for (int i = tid; i < kDCWaves * KT * kTile; i += kDCThreads) (&red[0][0][0])[i] = 0.f;
  __syncthreads();
  const int nv = s_nv;
  // lane p < KT: byte offset of the expert and natural slot of canonical position p. The
  // offset is added to the kernel argument, so the loads stay global (not flat) loads.
  const int pl = min(lane, KT - 1);
  const uint64_t voff = (uint64_t)s_sid[pl] * stride;
  const int vslot = s_slot[pl];
  auto base_of = [&](int p) {  // p wave-uniform
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)voff, p);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(voff >> 32), p);
    return packed + (((uint64_t)hi << 32) | lo);
  };

  // 4. this wave's first batch of weights. Steps s = p * nch + c (position p, chunk c) are
  // walked with carried (p, c) counters, all wave-uniform. Steps past this wave's range
  // repeat its last step (or step 0 when the token has no valid slot), so every load
  // reads packed data of a real expert.
  const int n_steps = nv * nch;
  const int s_begin = wv * n_steps / kDCWaves;
  const int s_end = (wv + 1) * n_steps / kDCWaves;
  const size_t tbase = (size_t)(row0 / kTile) * kTile * KBI;  // tile-major packed layout
  const int s_last = max(s_end - 1, 0);
  const int p_first = min(s_begin, s_last) / nch;
  const int c_first = min(s_begin, s_last) - p_first * nch;
  const int p_last = s_last / nch;
  const int c_last = s_last - p_last * nch;
  uint4 cd[kDCBatch];
  uint32_t sd[kDCBatch];
  auto load_batch = [&](int s0, int p, int c) {  // (p, c) = coordinates of step s0
#pragma unroll
    for (int q = 0; q < kDCBatch; ++q) {
      const bool in = s0 + q < s_end;
      const uint8_t* b = base_of(in ? p : p_last);
      const int cc = in ? c : c_last;
      const size_t w = tbase + ((4 * cc + g < KBI) ? 64 * cc + lane : 64 * cc);
      cd[q] = ld_stream(reinterpret_cast<const uint4*>(b + off_dc) + w);
      sd[q] = ld_scale(b + off_ds + w);
      if (++c == nch) {
        c = 0;
        ++p;
      }
    }
  };
  load_batch(s_begin, p_first, c_first);

  // 5. h into LDS
  const int dummy = hw + 4;
  {
    const int c0 = tid, c1 = tid + kDCThreads, c2 = tid + 2 * kDCThreads, c3 = tid + 3 * kDCThreads;
    smem[c0 < hw ? c0 : dummy] = hr0;
    if constexpr (HR > 1) smem[c1 < hw ? c1 : dummy] = hr1;
    if constexpr (HR > 2) smem[c2 < hw ? c2 : dummy] = hr2;
    if constexpr (HR > 3) smem[c3 < hw ? c3 : dummy] = hr3;
  }
  if (tid < 4) smem[hw + tid] = make_uint4(0, 0, 0, 0);
  __syncthreads();

  const char* lds = reinterpret_cast<const char*>(smem);
  const uint32_t zero_addr = (uint32_t)hw * 16u;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  int cur_p = p_first;
  int p = p_first, c = c_first;
  int hslot = __builtin_amdgcn_readlane(vslot, p_first) * hx;  // first h word of position p
  for (int s0 = s_begin; s0 < s_end; s0 += kDCBatch) {
#pragma unroll
    for (int q = 0; q < kDCBatch; ++q) {
      if (s0 + q < s_end) {  // wave-uniform
        if (p != cur_p) {  // wave-uniform: flush the finished slot
          if (lane < kTile) red[wv][cur_p][lane] = acc[0];
          acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
          cur_p = p;
          hslot = __builtin_amdgcn_readlane(vslot, p) * hx;
        }
        const bool bv = 4 * c + g < KBI;
        const uint32_t a_addr =
            (j16 == 0 && bv) ? (uint32_t)(hslot + 16 * c + 4 * g) * 16u : zero_addr;
        const uint4 wd = bv ? cd[q] : make_uint4(0, 0, 0, 0);
        const float fs = scale_operand(bv ? sd[q] : 127u);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(lds + a_addr + 16 * m));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, fp4x8_to_bf16(dword(wd, m), fs), acc, 0, 0, 0);
        }
        if (++c == nch) {
          c = 0;
          ++p;
        }
      }
    }
    if (s0 + kDCBatch < s_end) load_batch(s0 + kDCBatch, p, c);  // (p, c): step s0 + kDCBatch
  }
  if (s_begin < s_end && lane < kTile) red[wv][cur_p][lane] = acc[0];
  __syncthreads();
  if (tid < kTile && row0 + tid < H) {
    float yv = 0.f;
#pragma unroll
    for (int p = 0; p < KT; ++p) {
      if (p < nv) {
        float sp = 0.f;
#pragma unroll
        for (int w = 0; w < kDCWaves; ++w) sp += red[w][p][tid];
        yv += s_w[p] * sp;
      }
    }
    y[(size_t)t * H + row0 + tid] = f32_to_bf16_rne(yv);
  }
}

// One thread per (row, block) of one matrix: the FP4 decode of the FFN kernels themselves
// (fp4x8_to_bf16 with scale_operand, the conversion feeding their matrix-core B operands),
// each bf16 result widened to fp32 (exactly) and written out row-major [rows x K].
__global__ __launch_bounds__(256) void debug_dequant_kernel(const uint4* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            int rows, int kb, float* __restrict__ out) {
  const long b = (long)blockIdx.x * 256 + threadIdx.x;
  if (b >= (long)rows * kb) return;
  const int row = (int)(b / kb);
  const int blk = (int)(b - (long)row * kb);
  const long v = (long)(row / 16) * 16 * kb + 64L * (blk / 4) + 16 * (blk % 4) + (row % 16);
  const uint4 c = codes[v];
  const float s = scale_operand(scales[v]);
  float* o = out + b * kBlock;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const bf16x8_t d = fp4x8_to_bf16(dword(c, m), s);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[8 * m + i] = (float)d[i];
  }
}

template <int XR>
hipError_t gate_up_launch_xr(const uint16_t* x, const int32_t* ids, int T, int k,
                             const uint8_t* packed, int n_experts, int H, int I, uint16_t* hbuf,
                             hipStream_t s) {
  const PackedLayout L = packed_layout(H, I);
  const long tiles_per_pair = (I + kTile - 1) / kTile;
  const long blocks = (long)T * k * tiles_per_pair;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  const uint32_t lds = (uint32_t)((H / 8 + 4) * 16);
  return launch_kernel(kKindGateUp, gate_up_kernel<XR>, dim3((unsigned)blocks), dim3(kGUThreads),
                       lds, s, x, ids, k, packed, L.stride, L.m[0].codes, L.m[1].codes,
                       L.m[0].scales, L.m[1].scales, n_experts, H, I, (int)tiles_per_pair, hbuf);
}

template <int KT, int HR>
hipError_t down_launch_hr(const int32_t* ids, const float* w, int T, const uint8_t* packed,
                          int n_experts, int H, int I, const uint16_t* hbuf, uint16_t* y,
                          hipStream_t s) {
  const PackedLayout L = packed_layout(H, I);
  const long tiles = H / kTile;
  const long blocks = (long)T * tiles;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  const uint32_t lds = (uint32_t)(((size_t)KT * I / 8 + 5) * 16);
  // allow more than 64 KB of LDS per workgroup (the device has 160 KB per CU)
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(down_combine_kernel<KT, HR>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kMaxLdsH + 80));
  if (attr != hipSuccess) return attr;
  return launch_kernel(kKindDownCombine, down_combine_kernel<KT, HR>, dim3((unsigned)blocks),
                       dim3(kDCThreads), lds, s, ids, w, T, packed, L.stride, L.m[2].codes,
                       L.m[2].scales, n_experts, H, I, (int)tiles, hbuf, y);
}

template <int KT>
hipError_t down_launch(const int32_t* ids, const float* w, int T, const uint8_t* packed,
                       int n_experts, int H, int I, const uint16_t* hbuf, uint16_t* y,
                       hipStream_t s) {
  constexpr int kMaxRounds = (kMaxLdsH / 16 + kDCThreads - 1) / kDCThreads;
  const int rounds = (KT * I / 8 + kDCThreads - 1) / kDCThreads;
#define MOE_FP4_DC_LAUNCH(R) \
  return down_launch_hr<KT, R>(ids, w, T, packed, n_experts, H, I, hbuf, y, s)
  if (rounds <= 1) MOE_FP4_DC_LAUNCH(1);
  if (rounds <= 2) MOE_FP4_DC_LAUNCH(2);
  if (rounds <= 4) MOE_FP4_DC_LAUNCH(4);
  MOE_FP4_DC_LAUNCH((kMaxRounds > 4 ? kMaxRounds : 4));
#undef MOE_FP4_DC_LAUNCH
}

}  // namespace

hipError_t launch_gate_up(const uint16_t* x, const int32_t* ids, int T, int k, const uint8_t* packed,
                          int n_experts, int hidden, int inter, uint16_t* hbuf, hipStream_t s) {
  const int rounds = (hidden / 8 + kGUThreads - 1) / kGUThreads;
#define MOE_FP4_GU_LAUNCH(R) \
  return gate_up_launch_xr<R>(x, ids, T, k, packed, n_experts, hidden, inter, hbuf, s)
  if (rounds <= 1) MOE_FP4_GU_LAUNCH(1);
  if (rounds <= 2) MOE_FP4_GU_LAUNCH(2);
  if (rounds <= 4) MOE_FP4_GU_LAUNCH(4);
  MOE_FP4_GU_LAUNCH(kMaxDim / 8 / kGUThreads);
#undef MOE_FP4_GU_LAUNCH
}

hipError_t launch_down_combine(const int32_t* ids, const float* w, int T, int k,
                               const uint8_t* packed, int n_experts, int hidden, int inter,
                               const uint16_t* hbuf, uint16_t* y, hipStream_t s) {
  switch (k) {
    case 1: return down_launch<1>(ids, w, T, packed, n_experts, hidden, inter, hbuf, y, s);
    case 2: return down_launch<2>(ids, w, T, packed, n_experts, hidden, inter, hbuf, y, s);
    case 3: return down_launch<3>(ids, w, T, packed, n_experts, hidden, inter, hbuf, y, s);
    case 4: return down_launch<4>(ids, w, T, packed, n_experts, hidden, inter, hbuf, y, s);
    case 5: return down_launch<5>(ids, w, T, packed, n_experts, hidden, inter, hbuf, y, s);
    case 6: return down_launch<6>(ids, w, T, packed, n_experts, hidden, inter, hbuf, y, s);
    case 7: return down_launch<7>(ids, w, T, packed, n_experts, hidden, inter, hbuf, y, s);
    case 8: return down_launch<8>(ids, w, T, packed, n_experts, hidden, inter, hbuf, y, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_debug_dequant(const uint8_t* packed, int hidden, int inter, int expert,
                                int matrix, float* out, hipStream_t s) {
  const PackedLayout L = packed_layout(hidden, inter);
  const MatLayout& M = L.m[matrix];
  const uint8_t* base = packed + (size_t)expert * L.stride;
  const long n_blocks = (long)M.rows * M.kb;
  const long grid = (n_blocks + 255) / 256;
  debug_dequant_kernel<<<dim3((unsigned)grid), dim3(256), 0, s>>>(
      reinterpret_cast<const uint4*>(base + M.codes), base + M.scales, M.rows, M.kb, out);
  return hipGetLastError();
}

}  // namespace moe_fp4
