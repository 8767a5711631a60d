// Internal declarations shared by the HIP translation units of the library.
// Device code targets gfx950 (CDNA4) only: 64-lane wavefronts, the FP4 -> bf16 scaled
// conversion and the bf16 dot2 instruction.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe_fp4 {

constexpr int kBlock = 32;        // elements per ue8m0 scale block along K
constexpr int kMaxK = 8;          // max experts per token
constexpr int kMaxDim = 16384;    // max hidden / inter
constexpr int kMaxLdsH = 65536;   // bytes of LDS for the k staged h vectors of one token
constexpr int kMaxExpertsTopk = 2048;  // max experts for the top-k selection kernel

// Kernel kinds for timing (same values as MOE_FP4_KERNEL_* in the public header).
enum KernelKind { kKindPack = 0, kKindRouterGemv = 1, kKindTopk = 2, kKindGateUp = 3,
                  kKindDownCombine = 4, kKindRouteDecode = 5, kKindBatchedSort = 6,
                  kKindBatchedQuant = 7, kKindBatchedGateUp = 8, kKindBatchedDown = 9,
                  kKindBatchedCombine = 10, kKindNorm = 11,
                  kKindProbeStream = 12, kKindProbeMfma = 13, kKindSmallGateUp = 14,
                  kKindSmallDown = 15, kKindFp8Gemv = 16, kKindPrefetch = 17 };

// ----------------------------------------------------------------------------------------
// Packed expert layout (the output of moe_fp4_pack). An expert is three matrices (gate
// [I x H], up [I x H], down [H x I]; rows x K). Each matrix is stored tile-major: its rows
// (padded to a multiple of 16 with zero codes and scale byte 127) form 16-row tiles, K
// forms 128-element chunks (4 scale blocks), and for every (tile, chunk) the 16-byte code
// blocks are laid out as [block-in-chunk g][row-in-tile j], so the 64 lanes of a
// wavefront (lane = 16 g + j) read one contiguous 1 KB word per load. The last chunk of a
// row holds only the blocks that exist (K need not be a multiple of 128); its words keep
// the same [g][j] order. Scale bytes follow the same order, one byte per block: 64
// contiguous bytes per (tile, chunk).
//   code word  (tile, c, g, j) at  tile * 16 * KB + 64 c + 16 g + j   (16-byte units)
//   scale byte (tile, c, g, j) at  tile * 16 * KB + 64 c + 16 g + j   (bytes)
// with KB = K / 32. Codes of the three matrices come first, then their scales, each
// region 256-byte aligned; the expert stride is a multiple of 256.
// ----------------------------------------------------------------------------------------
struct MatLayout {
  size_t codes;   // byte offset of the code region inside one expert
  size_t scales;  // byte offset of the scale region
  int rows;       // rows of the matrix
  int tiles;      // 16-row tiles
  int kb;         // scale blocks per row (K / 32)
};

struct PackedLayout {
  MatLayout m[3];  // gate, up, down
  size_t stride;   // bytes per expert
};

inline size_t align_up256(size_t v) { return (v + 255) / 256 * 256; }

inline PackedLayout packed_layout(int hidden, int inter) {
  PackedLayout L;
  const int rows[3] = {inter, inter, hidden};
  const int kdim[3] = {hidden, hidden, inter};
  size_t off = 0;
  for (int i = 0; i < 3; ++i) {
    L.m[i].rows = rows[i];
    L.m[i].tiles = (rows[i] + 15) / 16;
    L.m[i].kb = kdim[i] / kBlock;
    L.m[i].codes = off;
    off += align_up256((size_t)L.m[i].tiles * 16 * L.m[i].kb * 16);
  }
  for (int i = 0; i < 3; ++i) {
    L.m[i].scales = off;
    off += align_up256((size_t)L.m[i].tiles * 16 * L.m[i].kb);
  }
  L.stride = align_up256(off);
  return L;
}

// Kernel timing. When timing is enabled, timing_slot hands out a pair of events for one
// launch of kernel `kind`; the launch passes them to hipExtLaunchKernel, which stamps them
// with the dispatch's own start and end times.
bool timing_slot(int kind, hipEvent_t* start, hipEvent_t* stop);

template <typename... KArgs, typename... Args>
hipError_t launch_kernel(int kind, void (*kernel)(KArgs...), dim3 grid, dim3 block,
                         uint32_t shmem, hipStream_t s, Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (timing_slot(kind, &e0, &e1)) {
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, e0, e1, 0, static_cast<KArgs>(args)...);
  } else {
    kernel<<<grid, block, shmem, s>>>(static_cast<KArgs>(args)...);
  }
  return hipGetLastError();
}

// Kernel launchers. Each returns hipSuccess or the launch error.
hipError_t launch_pack(const uint8_t* codes, const uint8_t* scales, int n_experts, int hidden,
                       int inter, uint8_t* packed, hipStream_t s);

hipError_t launch_router_gemv(const uint16_t* x, const uint16_t* wr, int T, int hidden,
                              int n_experts, double* logits, hipStream_t s);

// Batch-1 routing in one launch (GEMV + top-k); sync: route_decode_sync_words(E) words
// that persist between calls (their initial contents do not matter).
hipError_t launch_route_decode(const uint16_t* x, const uint16_t* wr, int hidden, int n_experts,
                               int k, uint32_t* sync, double* logits, int32_t* ids, float* w,
                               hipStream_t s);
int route_decode_sync_words(int n_experts);
// Bound of the batch-1 route's wait for each logit record (polls; the default unless set by
// moe_fp4_debug_route_spin_limit), the failure-mark query and the clearing of the area.
unsigned route_spin_limit();
void set_route_spin_limit(long long polls);
hipError_t launch_route_status(const uint32_t* sync, int32_t* status, hipStream_t s);
hipError_t launch_route_reset(uint32_t* sync, size_t bytes, hipStream_t s);
// The same with the router input computed in the kernel from a residual stream (one token):
// r_out = r_in + y_prev, x_out = bf16(r_out / rms) with the standalone norm kernel's bits.
hipError_t launch_route_decode_norm(const float* r_in, const uint16_t* y_prev, float* r_out,
                                    uint16_t* x_out, float eps, const uint16_t* wr, int hidden,
                                    int n_experts, int k, uint32_t* sync, double* logits,
                                    int32_t* ids, float* w, hipStream_t s);

hipError_t launch_topk_f64(const double* logits, int T, int n_experts, int k, int32_t* ids,
                           float* w, hipStream_t s);
hipError_t launch_topk_f32(const float* logits, int T, int n_experts, int k, int32_t* ids,
                           float* w, hipStream_t s);

hipError_t launch_gate_up(const uint16_t* x, const int32_t* ids, int T, int k, const uint8_t* packed,
                          int n_experts, int hidden, int inter, uint16_t* hbuf, hipStream_t s);

hipError_t launch_down_combine(const int32_t* ids, const float* w, int T, int k,
                               const uint8_t* packed, int n_experts, int hidden, int inter,
                               const uint16_t* hbuf, uint16_t* y, hipStream_t s);

// ----------------------------------------------------------------------------------------
// Batched path: pairs grouped by expert, grouped GEMM on the block-scaled matrix cores.
// Workspace regions (byte offsets, 256-aligned) for T tokens:
//   offsets [E+1], perm [T k], M-block table (expert, first sorted row) [nb_max each],
//   n_blocks [1], the split sort's per-workgroup counts [256 x E],
//   x as MX hi / lo [T x Hp bytes reserved each: 24 bytes per 32-block as two E2M3 terms,
//   32 as one E4M3 term] + scales [T x Hp/32] each,
//   h the same over [T k x Ip], per-pair weighted y_e fp32 [T k x H].
// Hp, Ip: hidden, inter rounded up to 128.
// ----------------------------------------------------------------------------------------
constexpr int kBlockRows = 64;  // rows of one expert's group per GEMM workgroup

struct BatchedLayout {
  size_t offsets, perm, blk_expert, blk_row0, n_blocks, sort_cnt;
  size_t xhi, xlo, xshi, xslo, hhi, hlo, hshi, hslo, ypair;
  size_t bytes, nb_max;
  int Hp, Ip;
};

BatchedLayout batched_layout(int T, int k, int n_experts, int hidden, int inter);

// terms: 2 = x and h as two MX terms (hi + lo; E2M3 by default), 1 = one E4M3 term (hi only)
hipError_t launch_batched_ffn(const uint16_t* x, const int32_t* ids, const float* w, int T, int k,
                              const uint8_t* packed, int n_experts, int hidden, int inter,
                              uint16_t* y, void* workspace, int terms, hipStream_t s);

// Layer chaining helpers (multi-layer decode harness).
hipError_t launch_residual_init(const uint16_t* x, float* r, int T, int hidden, hipStream_t s);
hipError_t launch_residual_rmsnorm(const float* r_in, const uint16_t* y, float* r_out, uint16_t* x,
                                   int T, int hidden, float eps, hipStream_t s);

// Small-M FFN (a few tokens; pairs that chose one expert share its weight stream): gate/up
// and down per group of up to small_m_rows(...) pairs, then the fixed-order combine.
// Workspace: small_m_workspace_bytes(...). T * k <= 256.
int small_m_rows(int T, int hidden, int inter);
size_t small_m_workspace_bytes(int T, int k, int hidden, int inter);
hipError_t launch_small_m_ffn(const uint16_t* x, const int32_t* ids, const float* w, int T, int k,
                              const uint8_t* packed, int n_experts, int hidden, int inter,
                              void* workspace, uint16_t* y, hipStream_t s);
// The grouped path's combine: y[t] = sum over t's valid slots, in canonical order, of the
// pair rows ypair [T*k x hidden] fp32 (already weighted), rounded to bf16.
hipError_t launch_combine_pairs(const int32_t* ids, const float* w, int T, int k, int n_experts,
                                int hidden, const float* ypair, uint16_t* y, hipStream_t s);

// Dense FP8 (E4M3) matrices [rows x cols] with one fp32 multiplier per 128 x 128 block:
// load-time packing, y = x W^T, and the SwiGLU pair h = silu(x Wg^T) * (x Wu^T).
size_t fp8_packed_bytes(int rows, int cols);
hipError_t launch_fp8_pack(const uint8_t* codes, const float* scale_inv, int rows, int cols,
                           uint8_t* packed, hipStream_t s);
hipError_t launch_fp8_linear(const uint16_t* x, int T, const uint8_t* packed, int rows, int cols,
                             uint16_t* y, hipStream_t s);
hipError_t launch_fp8_swiglu(const uint16_t* x, int T, const uint8_t* gate, const uint8_t* up,
                             int inter, int hidden, uint16_t* h, hipStream_t s);

// Measurement kernels: a streaming read of `bytes` bytes, and n_workgroups x 4 wavefronts
// each issuing iters x probe_mfma_chains() block-scaled 16x16x128 MFMAs (B FP4, A FP4 when
// fmt_a == 4 else FP8 E4M3).
hipError_t launch_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_probe_mfma_loop(int fmt_a, int n_workgroups, int iters, uint32_t* sink,
                                  hipStream_t s);
int probe_mfma_chains();

// The grouped path's activation quantisation of x [T x H] (terms 1: one E4M3 term; 2: two E2M3 terms)
// decoded back to fp32 out [T x H]; workspace debug_act_quant_bytes(T, H).
size_t debug_act_quant_bytes(int T, int H);
hipError_t launch_debug_act_quant(const uint16_t* x, int T, int H, int terms, void* ws,
                                  float* out, hipStream_t s);

hipError_t launch_debug_dequant(const uint8_t* packed, int hidden, int inter, int expert,
                                int matrix, float* out, hipStream_t s);

// Reads the chosen matrices (bit 0 gate, 1 up, 2 down; codes and scales) of the experts
// ids[0 .. n_ids - 1] of a packed buffer with cached loads (ids outside [0, n_experts)
// skipped); writes nothing except, practically never, one word of sink.
hipError_t launch_prefetch_experts(const int32_t* ids, int n_ids, const uint8_t* packed,
                                   int n_experts, int hidden, int inter, int matrices,
                                   uint32_t* sink, hipStream_t s);

hipError_t launch_validate_ids(const int32_t* ids, int T, int k, int n_experts, int32_t* bad,
                               hipStream_t s);

}  // namespace moe_fp4
