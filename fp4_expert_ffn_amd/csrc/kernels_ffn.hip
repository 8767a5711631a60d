// Routed expert FFN, GEMV form: every (token, slot) pair streams its expert's rows.
//
// Stage 1 (gate_up): g = W_gate[e] x, u = W_up[e] x, h = silu(g) * u, for every pair
//   (t, j) with a valid id; h is written as bf16 to the workspace, natural order [pair][I].
// Stage 2 (down_combine): for every token t and output row n,
//   y[t, n] = sum over the token's valid slots, in ascending expert id, of
//             w_j * (W_down[e_j] h_j)[n],
//   with the k h vectors of the token staged in LDS; y is written as bf16.
//
// The FP4 weights are read once per pair with 16-byte loads: a wave's 64 lanes read 64
// consecutive 32-code blocks (1 KB) of a row per load instruction. Each block is
// dequantised in registers (hardware FP4 -> bf16 conversion, exact), dotted with the
// activations in fp32 (bf16 dot2), then multiplied by its ue8m0 scale 2^(e-127). The
// weights are never expanded in memory: storage format and compute format differ only in
// registers ([A100-FP4], section 「FP4非対応」という言葉を疑う).
#include "moe_fp4_device.hpp"
#include "moe_fp4_internal.hpp"

namespace moe_fp4 {

namespace {

constexpr int kThreads = 256;  // 4 wavefronts per workgroup
constexpr int kWaves = kThreads / 64;

// ---------------------------------------------------------------------------------------
// Stage 1: gate/up/SiLU. One wave owns `rows_per_wave` consecutive rows of one pair.
// LPR lanes per row, BPL blocks per lane; UNR row-iterations are loaded before any is
// consumed so that UNR * BPL * 2 16-byte loads per lane are in flight.
// ---------------------------------------------------------------------------------------
template <int LPR, int BPL, int UNR>
__global__ __launch_bounds__(kThreads) void gate_up_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids, int n_pairs, int k,
    const uint8_t* __restrict__ packed, size_t stride, size_t off_gc, size_t off_uc,
    size_t off_gs, size_t off_us, int n_experts, int H, int I, int rows_per_wave,
    int tasks_per_pair, uint16_t* __restrict__ hbuf) {
  constexpr int RPI = 64 / LPR;  // rows per iteration
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int pair = wave / tasks_per_pair;
  if (pair >= n_pairs) return;  // whole wave leaves together
  const int e = ids[pair];
  if (e < 0 || e >= n_experts) return;
  const int t = pair / k;
  const int row0 = (wave - pair * tasks_per_pair) * rows_per_wave;
  const int row_end = min(row0 + rows_per_wave, I);
  const int sub = lane / LPR;
  const int li = lane - sub * LPR;
  const int KB = H / kBlock;

  // Activations for this lane's blocks, kept in registers for all rows.
  uint4 xa[BPL][4];
  const uint4* xv = reinterpret_cast<const uint4*>(x + (size_t)t * H);
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int b = li + i * LPR;
#pragma unroll
    for (int q = 0; q < 4; ++q) xa[i][q] = (b < KB) ? xv[b * 4 + q] : make_uint4(0, 0, 0, 0);
  }

  const uint8_t* base = packed + (size_t)e * stride;
  const uint4* gcodes = reinterpret_cast<const uint4*>(base + off_gc);
  const uint4* ucodes = reinterpret_cast<const uint4*>(base + off_uc);
  const uint8_t* gscales = base + off_gs;
  const uint8_t* uscales = base + off_us;
  const int n_iter = (row_end - row0 + RPI - 1) / RPI;

  for (int it0 = 0; it0 < n_iter; it0 += UNR) {
    uint4 cg[UNR][BPL], cu[UNR][BPL];
    uint32_t sg[UNR][BPL], su[UNR][BPL];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int r = row0 + (it0 + u) * RPI + sub;
      const bool rv = r < row_end;
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        const int b = li + i * LPR;
        if (rv && b < KB) {
          const size_t blk = (size_t)r * KB + b;
          cg[u][i] = gcodes[blk];
          cu[u][i] = ucodes[blk];
          sg[u][i] = gscales[blk];
          su[u][i] = uscales[blk];
        } else {
          cg[u][i] = make_uint4(0, 0, 0, 0);
          cu[u][i] = make_uint4(0, 0, 0, 0);
          sg[u][i] = 127u;
          su[u][i] = 127u;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float ag = 0.f, au = 0.f;
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        ag += ue8m0_to_f32(sg[u][i]) *
              fp4_block_dot(cg[u][i], xa[i][0], xa[i][1], xa[i][2], xa[i][3]);
        au += ue8m0_to_f32(su[u][i]) *
              fp4_block_dot(cu[u][i], xa[i][0], xa[i][1], xa[i][2], xa[i][3]);
      }
      ag = group_sum<LPR>(ag);
      au = group_sum<LPR>(au);
      const int r = row0 + (it0 + u) * RPI + sub;
      if (li == 0 && r < row_end) {
        hbuf[(size_t)pair * I + r] = f32_to_bf16_rne(silu_f32(ag) * au);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Stage 2: down projection and weighted combine. One workgroup owns `rows_per_block`
// output rows of one token; its waves take RPI rows at a time.
// LDS holds the token's h vectors as bf16 in a layout where, for part q (elements
// 8q..8q+7 of a block) of block b of slot j, the 16 bytes sit at ((j*4 + q) * KBI + b):
// the lanes of a row group read consecutive 16-byte words.
// ---------------------------------------------------------------------------------------
template <int LPR, int BPL>
__global__ __launch_bounds__(kThreads) void down_combine_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ wts, int T, int k,
    const uint8_t* __restrict__ packed, size_t stride, size_t off_dc, size_t off_ds,
    int n_experts, int H, int I, int rows_per_block, int chunks_per_token,
    const uint16_t* __restrict__ hbuf, uint16_t* __restrict__ y) {
  extern __shared__ uint4 lds_h[];
  constexpr int RPI = 64 / LPR;
  const int t = blockIdx.x / chunks_per_token;
  const int n0 = (blockIdx.x - t * chunks_per_token) * rows_per_block;
  const int n_end = min(n0 + rows_per_block, H);
  const int KBI = I / kBlock;

  // Canonical slot order: ascending expert id, then ascending weight bits; invalid ids
  // dropped. Ranks are computed with static indexing only (no private-memory arrays).
  int ev[kMaxK];
  uint32_t wb[kMaxK];
  bool ok[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    ev[j] = -1;
    wb[j] = 0u;
    ok[j] = false;
    if (j < k) {
      ev[j] = ids[(size_t)t * k + j];
      wb[j] = __float_as_uint(wts[(size_t)t * k + j]);
      ok[j] = ev[j] >= 0 && ev[j] < n_experts;
    }
  }
  int sid[kMaxK], sslot[kMaxK];
  float sw[kMaxK];
  int nv = 0;
#pragma unroll
  for (int p = 0; p < kMaxK; ++p) {
    sid[p] = 0;
    sslot[p] = 0;
    sw[p] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    int rank = 0;
#pragma unroll
    for (int i = 0; i < kMaxK; ++i) {
      const bool before = ev[i] < ev[j] || (ev[i] == ev[j] && (wb[i] < wb[j] || (wb[i] == wb[j] && i < j)));
      rank += (ok[i] && before) ? 1 : 0;
    }
    nv += ok[j] ? 1 : 0;
#pragma unroll
    for (int p = 0; p < kMaxK; ++p) {
      if (ok[j] && rank == p) {
        sid[p] = ev[j];
        sslot[p] = j;
        sw[p] = __uint_as_float(wb[j]);
      }
    }
  }

  // Stage h of the valid slots into LDS.
  const int chunks = I / 8;  // 16-byte chunks per h vector
  for (int c = threadIdx.x; c < nv * chunks; c += kThreads) {
    const int j = c / chunks;
    const int cc = c - j * chunks;
    int slot = 0;
#pragma unroll
    for (int q = 0; q < kMaxK; ++q)
      if (q == j) slot = sslot[q];
    const uint4 v =
        reinterpret_cast<const uint4*>(hbuf + ((size_t)t * k + slot) * I)[cc];
    const int b = cc >> 2, q = cc & 3;
    lds_h[(j * 4 + q) * KBI + b] = v;
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int sub = lane / LPR;
  const int li = lane - sub * LPR;

  for (int nb = n0 + wv * RPI; nb < n_end; nb += kWaves * RPI) {
    const int n = nb + sub;
    const bool rv = n < n_end;
    uint4 cd[kMaxK][BPL];
    uint32_t sd[kMaxK][BPL];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < nv) {
        const uint8_t* base = packed + (size_t)sid[j] * stride;
        const uint4* dcodes = reinterpret_cast<const uint4*>(base + off_dc);
        const uint8_t* dscales = base + off_ds;
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
          const int b = li + i * LPR;
          if (rv && b < KBI) {
            const size_t blk = (size_t)n * KBI + b;
            cd[j][i] = dcodes[blk];
            sd[j][i] = dscales[blk];
          } else {
            cd[j][i] = make_uint4(0, 0, 0, 0);
            sd[j][i] = 127u;
          }
        }
      }
    }
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < nv) {
        float pj = 0.f;
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
          const int b = li + i * LPR;
          if (b < KBI) {
            const uint4 h0 = lds_h[(j * 4 + 0) * KBI + b];
            const uint4 h1 = lds_h[(j * 4 + 1) * KBI + b];
            const uint4 h2 = lds_h[(j * 4 + 2) * KBI + b];
            const uint4 h3 = lds_h[(j * 4 + 3) * KBI + b];
            pj += ue8m0_to_f32(sd[j][i]) * fp4_block_dot(cd[j][i], h0, h1, h2, h3);
          }
        }
        acc += sw[j] * pj;
      }
    }
    acc = group_sum<LPR>(acc);
    if (li == 0 && rv) y[(size_t)t * H + n] = f32_to_bf16_rne(acc);
  }
}

template <int LPR, int BPL>
hipError_t gate_up_dispatch(const uint16_t* x, const int32_t* ids, int T, int k,
                            const uint8_t* packed, int n_experts, int H, int I,
                            uint16_t* hbuf, hipStream_t s) {
  constexpr int UNR = (BPL <= 2) ? 4 : 2;
  constexpr int RPI = 64 / LPR;
  const PackedLayout L = packed_layout(H, I);
  const long n_pairs = (long)T * k;
  // Rows per wave: enough waves to cover the GPU several times over, in multiples of the
  // rows one unrolled step covers.
  const long step = (long)RPI * UNR;
  long rpw = (n_pairs * I + 4095) / 4096;
  rpw = (rpw + step - 1) / step * step;
  if (rpw < step) rpw = step;
  if (rpw > 64 && rpw > step) rpw = (64 / step > 0 ? 64 / step : 1) * step;
  const long tasks_per_pair = (I + rpw - 1) / rpw;
  const long waves = n_pairs * tasks_per_pair;
  const long blocks = (waves + kWaves - 1) / kWaves;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gate_up_kernel<LPR, BPL, UNR>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     s, x, ids, (int)n_pairs, k, packed, L.stride, L.gate_codes, L.up_codes,
                     L.gate_scales, L.up_scales, n_experts, H, I, (int)rpw, (int)tasks_per_pair,
                     hbuf);
  return hipGetLastError();
}

template <int LPR, int BPL>
hipError_t down_dispatch(const int32_t* ids, const float* w, int T, int k, const uint8_t* packed,
                         int n_experts, int H, int I, const uint16_t* hbuf, uint16_t* y,
                         hipStream_t s) {
  constexpr int RPI = 64 / LPR;
  const PackedLayout L = packed_layout(H, I);
  // Rows per workgroup: about 256 workgroups in total (one per CU) for a single token,
  // growing with T so that the h staging (k * I * 2 bytes per workgroup) is amortised.
  const long minr = (long)kWaves * RPI;
  long rpb = ((long)T * H + 255) / 256;
  rpb = (rpb + minr - 1) / minr * minr;
  if (rpb > H) rpb = H;
  const long chunks = (H + rpb - 1) / rpb;
  const long blocks = (long)T * chunks;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  const size_t lds = (size_t)k * I * 2;
  hipLaunchKernelGGL((down_combine_kernel<LPR, BPL>), dim3((unsigned)blocks), dim3(kThreads),
                     lds, s, ids, w, T, k, packed, L.stride, L.down_codes, L.down_scales,
                     n_experts, H, I, (int)rpb, (int)chunks, hbuf, y);
  return hipGetLastError();
}

#define MOE_FP4_ROWMAP_SWITCH(FN, ...)                                 \
  switch (rm.lpr * 16 + rm.bpl) {                                      \
    case 64 * 16 + 1: return FN<64, 1>(__VA_ARGS__);                   \
    case 64 * 16 + 2: return FN<64, 2>(__VA_ARGS__);                   \
    case 64 * 16 + 3: return FN<64, 3>(__VA_ARGS__);                   \
    case 64 * 16 + 4: return FN<64, 4>(__VA_ARGS__);                   \
    case 64 * 16 + 5: return FN<64, 5>(__VA_ARGS__);                   \
    case 64 * 16 + 6: return FN<64, 6>(__VA_ARGS__);                   \
    case 64 * 16 + 7: return FN<64, 7>(__VA_ARGS__);                   \
    case 64 * 16 + 8: return FN<64, 8>(__VA_ARGS__);                   \
    case 32 * 16 + 1: return FN<32, 1>(__VA_ARGS__);                   \
    case 32 * 16 + 2: return FN<32, 2>(__VA_ARGS__);                   \
    case 32 * 16 + 3: return FN<32, 3>(__VA_ARGS__);                   \
    case 32 * 16 + 4: return FN<32, 4>(__VA_ARGS__);                   \
    case 16 * 16 + 1: return FN<16, 1>(__VA_ARGS__);                   \
    case 16 * 16 + 2: return FN<16, 2>(__VA_ARGS__);                   \
    case 16 * 16 + 3: return FN<16, 3>(__VA_ARGS__);                   \
    case 16 * 16 + 4: return FN<16, 4>(__VA_ARGS__);                   \
    case 8 * 16 + 1: return FN<8, 1>(__VA_ARGS__);                     \
    case 8 * 16 + 2: return FN<8, 2>(__VA_ARGS__);                     \
    case 8 * 16 + 3: return FN<8, 3>(__VA_ARGS__);                     \
    case 8 * 16 + 4: return FN<8, 4>(__VA_ARGS__);                     \
    default: return hipErrorInvalidValue;                              \
  }

// One thread per 32-element block: the decode of the FFN kernels, written out to memory.
__global__ __launch_bounds__(kThreads) void debug_dequant_kernel(const uint4* __restrict__ codes,
                                                                 const uint8_t* __restrict__ scales,
                                                                 long n_blocks,
                                                                 float* __restrict__ out) {
  const long b = (long)blockIdx.x * kThreads + threadIdx.x;
  if (b >= n_blocks) return;
  const uint4 c = codes[b];
  const float s = ue8m0_to_f32(scales[b]);
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float* o = out + b * kBlock;
#define MOE_FP4_DQ_WORD(Q)                                                        \
  {                                                                               \
    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[Q], 1.0f, 0); \
    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[Q], 1.0f, 1); \
    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[Q], 1.0f, 2); \
    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[Q], 1.0f, 3); \
    o[Q * 8 + 0] = (float)p0.x * s;                                               \
    o[Q * 8 + 1] = (float)p0.y * s;                                               \
    o[Q * 8 + 2] = (float)p1.x * s;                                               \
    o[Q * 8 + 3] = (float)p1.y * s;                                               \
    o[Q * 8 + 4] = (float)p2.x * s;                                               \
    o[Q * 8 + 5] = (float)p2.y * s;                                               \
    o[Q * 8 + 6] = (float)p3.x * s;                                               \
    o[Q * 8 + 7] = (float)p3.y * s;                                               \
  }
  MOE_FP4_DQ_WORD(0)
  MOE_FP4_DQ_WORD(1)
  MOE_FP4_DQ_WORD(2)
  MOE_FP4_DQ_WORD(3)
#undef MOE_FP4_DQ_WORD
}

}  // namespace

hipError_t launch_debug_dequant(const uint8_t* packed, int hidden, int inter, int expert,
                                int matrix, float* out, hipStream_t s) {
  const PackedLayout L = packed_layout(hidden, inter);
  const size_t coff[3] = {L.gate_codes, L.up_codes, L.down_codes};
  const size_t soff[3] = {L.gate_scales, L.up_scales, L.down_scales};
  const uint8_t* base = packed + (size_t)expert * L.stride;
  const long n_blocks = (long)hidden * inter / kBlock;
  const long grid = (n_blocks + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(debug_dequant_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s,
                     reinterpret_cast<const uint4*>(base + coff[matrix]), base + soff[matrix],
                     n_blocks, out);
  return hipGetLastError();
}

hipError_t launch_gate_up(const uint16_t* x, const int32_t* ids, int T, int k,
                          const uint8_t* packed, int n_experts, int hidden, int inter,
                          uint16_t* hbuf, hipStream_t s) {
  const RowMap rm = choose_row_map(hidden / kBlock);
  MOE_FP4_ROWMAP_SWITCH(gate_up_dispatch, x, ids, T, k, packed, n_experts, hidden, inter, hbuf, s)
}

hipError_t launch_down_combine(const int32_t* ids, const float* w, int T, int k,
                               const uint8_t* packed, int n_experts, int hidden, int inter,
                               const uint16_t* hbuf, uint16_t* y, hipStream_t s) {
  const RowMap rm = choose_row_map(inter / kBlock);
  MOE_FP4_ROWMAP_SWITCH(down_dispatch, ids, w, T, k, packed, n_experts, hidden, inter, hbuf, y, s)
}

}  // namespace moe_fp4
