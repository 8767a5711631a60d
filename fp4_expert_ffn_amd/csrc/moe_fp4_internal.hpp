// Internal declarations shared by the HIP translation units of the library.
// Device code targets gfx950 (CDNA4) only: 64-lane wavefronts, the FP4 -> bf16 scaled
// conversion and the bf16 dot2 instruction.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe_fp4 {

constexpr int kBlock = 32;        // elements per ue8m0 scale block along K
constexpr int kMaxK = 8;          // max experts per token
constexpr int kMaxDim = 16384;    // max hidden / inter
constexpr int kMaxExpertsTopk = 2048;  // max experts for the top-k selection kernel
constexpr int kMaxLdsH = 65536;   // bytes of LDS for the k staged h vectors of one token

// ----------------------------------------------------------------------------------------
// Packed expert layout (the output of moe_fp4_pack). Per expert, at e * stride:
//   codes  gate [I x H/2] | up [I x H/2] | down [H x I/2]
//   scales gate [I x H/32] | up [I x H/32] | down [H x I/32]
// stride = code bytes + scale bytes rounded up to 256.
// ----------------------------------------------------------------------------------------
struct PackedLayout {
  size_t gate_codes, up_codes, down_codes;   // byte offsets inside one expert
  size_t gate_scales, up_scales, down_scales;
  size_t stride;                             // bytes per expert
};

inline PackedLayout packed_layout(int hidden, int inter) {
  PackedLayout L;
  const size_t hi = (size_t)hidden * (size_t)inter;
  L.gate_codes = 0;
  L.up_codes = hi / 2;
  L.down_codes = hi;
  L.gate_scales = 3 * hi / 2;
  L.up_scales = L.gate_scales + hi / kBlock;
  L.down_scales = L.up_scales + hi / kBlock;
  const size_t bytes = L.down_scales + hi / kBlock;
  L.stride = (bytes + 255) / 256 * 256;
  return L;
}

// Lane mapping of a K-long row: LPR lanes share one row, lane li owns the 32-element
// blocks li, li + LPR, ..., li + (BPL-1) * LPR. 64 / LPR rows are processed at once.
struct RowMap {
  int lpr;
  int bpl;
};

// Pick (LPR, BPL) for kb = K / 32 blocks: the fewest idle lane slots, BPL <= 4 when
// possible, else LPR = 64 with BPL <= 8. Returns bpl = 0 if K is too large.
inline RowMap choose_row_map(int kb) {
  RowMap best{0, 0};
  double best_eff = -1.0;
  const int lprs[4] = {64, 32, 16, 8};
  for (int i = 0; i < 4; ++i) {
    const int lpr = lprs[i];
    const int bpl = (kb + lpr - 1) / lpr;
    if (bpl > 4) continue;
    const double eff = (double)kb / (double)(lpr * bpl);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = RowMap{lpr, bpl};
    }
  }
  if (best.bpl == 0) {
    const int bpl = (kb + 63) / 64;
    if (bpl <= 8) best = RowMap{64, bpl};
  }
  return best;
}

// Timing hooks (no-ops unless timing is enabled).
void timing_begin(int kind, hipStream_t s);
void timing_end(int kind, hipStream_t s);

// Kernel launchers. Each returns hipSuccess or the launch error.
hipError_t launch_pack(const uint8_t* codes, const uint8_t* scales, int n_experts, int hidden,
                       int inter, uint8_t* packed, hipStream_t s);

hipError_t launch_router_gemv(const uint16_t* x, const uint16_t* wr, int T, int hidden,
                              int n_experts, double* logits, hipStream_t s);

hipError_t launch_topk_f64(const double* logits, int T, int n_experts, int k, int32_t* ids,
                           float* w, hipStream_t s);
hipError_t launch_topk_f32(const float* logits, int T, int n_experts, int k, int32_t* ids,
                           float* w, hipStream_t s);

hipError_t launch_gate_up(const uint16_t* x, const int32_t* ids, int T, int k,
                          const uint8_t* packed, int n_experts, int hidden, int inter,
                          uint16_t* hbuf, hipStream_t s);

hipError_t launch_down_combine(const int32_t* ids, const float* w, int T, int k,
                               const uint8_t* packed, int n_experts, int hidden, int inter,
                               const uint16_t* hbuf, uint16_t* y, hipStream_t s);

hipError_t launch_debug_dequant(const uint8_t* packed, int hidden, int inter, int expert,
                                int matrix, float* out, hipStream_t s);

hipError_t launch_validate_ids(const int32_t* ids, int T, int k, int n_experts, int32_t* bad,
                               hipStream_t s);

}  // namespace moe_fp4
