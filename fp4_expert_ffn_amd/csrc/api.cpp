// C ABI of the routed FP4 expert FFN library: argument checks, workspace sizing, kernel
// dispatch on the caller's stream, and the optional kernel timing hooks.
#include <algorithm>
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <vector>

#include "moe_fp4.h"
#include "moe_fp4_internal.hpp"

using namespace moe_fp4;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool valid_dim(int d) { return d > 0 && d % kBlock == 0 && d <= kMaxDim; }

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

int from_hip(hipError_t e) { return e == hipSuccess ? MOE_FP4_OK : MOE_FP4_ERR_HIP; }

// ---------------------------------------------------------------------------------------
// Timing: pairs of events around each launch, kept per kernel kind until read.
// ---------------------------------------------------------------------------------------
struct TimingState {
  bool enabled = false;
  struct Rec {
    int kind;
    hipEvent_t start, stop;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> free_events;
};

TimingState& timing() {
  static TimingState st;
  return st;
}

hipEvent_t take_event() {
  TimingState& st = timing();
  if (!st.free_events.empty()) {
    hipEvent_t e = st.free_events.back();
    st.free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace moe_fp4 {

bool timing_slot(int kind, hipEvent_t* start, hipEvent_t* stop) {
  TimingState& st = timing();
  if (!st.enabled) return false;
  hipEvent_t a = take_event();
  if (!a) return false;
  hipEvent_t b = take_event();
  if (!b) {
    st.free_events.push_back(a);
    return false;
  }
  st.recs.push_back({kind, a, b});
  *start = a;
  *stop = b;
  return true;
}

}  // namespace moe_fp4

extern "C" {

int moe_fp4_version(void) { return 100; }

const char* moe_fp4_strerror(int status) {
  switch (status) {
    case MOE_FP4_OK: return "ok";
    case MOE_FP4_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size or k out of range)";
    case MOE_FP4_ERR_BAD_SHAPE: return "unsupported shape (hidden/inter must be multiples of 32, at most 16384; k*inter <= 32768)";
    case MOE_FP4_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
    case MOE_FP4_ERR_WORKSPACE: return "workspace or packed buffer too small";
    case MOE_FP4_ERR_HIP: return "HIP runtime or launch error";
    case MOE_FP4_ERR_TOO_LARGE: return "the call needs more memory than the static scratch of the no-allocation entry point (MOE_FP4_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

size_t moe_fp4_packed_expert_stride(int hidden, int inter) {
  if (!valid_dim(hidden) || !valid_dim(inter)) return 0;
  return packed_layout(hidden, inter).stride;
}

size_t moe_fp4_packed_bytes(int n_experts, int hidden, int inter) {
  if (n_experts <= 0) return 0;
  const size_t stride = moe_fp4_packed_expert_stride(hidden, inter);
  return stride * (size_t)n_experts;
}

int moe_fp4_pack(const uint8_t* codes, const uint8_t* scales, int n_experts, int hidden,
                 int inter, void* packed, size_t packed_bytes, void* stream) {
  if (!codes || !scales || !packed || n_experts <= 0) return MOE_FP4_ERR_INVALID_ARG;
  if (!valid_dim(hidden) || !valid_dim(inter)) return MOE_FP4_ERR_BAD_SHAPE;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(packed)) return MOE_FP4_ERR_MISALIGNED;
  if (packed_bytes < moe_fp4_packed_bytes(n_experts, hidden, inter)) return MOE_FP4_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip((launch_pack(codes, scales, n_experts, hidden, inter,
                                            static_cast<uint8_t*>(packed), s)));
}

// Route workspace: a 16 KB synchronisation area (kept between calls: the epoch word and one
// 16-byte logit record per expert for the batch-1 kernel), then fp64 logits.
constexpr size_t kRouteSyncBytes = 16384;

size_t moe_fp4_route_workspace_bytes(int T, int n_experts) {
  if (T < 0 || n_experts <= 0) return 0;
  return kRouteSyncBytes + align256((size_t)T * (size_t)n_experts * sizeof(double));
}

static int check_topk_args(int T, int n_experts, int k) {
  if (T < 0 || n_experts <= 0) return MOE_FP4_ERR_INVALID_ARG;
  if (k < 1 || k > kMaxK || k > n_experts) return MOE_FP4_ERR_INVALID_ARG;
  if (n_experts > kMaxExpertsTopk) return MOE_FP4_ERR_BAD_SHAPE;
  return MOE_FP4_OK;
}

static hipError_t route_impl(const uint16_t* x, const uint16_t* w_router, int T, int hidden,
                             int n_experts, int k, int32_t* topk_ids, float* topk_w,
                             void* workspace, hipStream_t s) {
  uint32_t* sync = static_cast<uint32_t*>(workspace);
  double* logits = reinterpret_cast<double*>(static_cast<uint8_t*>(workspace) + kRouteSyncBytes);
  if (T == 1 && (size_t)route_decode_sync_words(n_experts) * 4 <= kRouteSyncBytes)
    return launch_route_decode(x, w_router, hidden, n_experts, k, sync, logits, topk_ids, topk_w, s);
  hipError_t e = launch_router_gemv(x, w_router, T, hidden, n_experts, logits, s);
  if (e != hipSuccess) return e;
  return launch_topk_f64(logits, T, n_experts, k, topk_ids, topk_w, s);
}

int moe_fp4_route(const uint16_t* x, const uint16_t* w_router, int T, int hidden, int n_experts,
                  int k, int32_t* topk_ids, float* topk_w, void* workspace,
                  size_t workspace_bytes, void* stream) {
  if (!x || !w_router || !topk_ids || !topk_w || !workspace) return MOE_FP4_ERR_INVALID_ARG;
  int st = check_topk_args(T, n_experts, k);
  if (st != MOE_FP4_OK) return st;
  if (!valid_dim(hidden)) return MOE_FP4_ERR_BAD_SHAPE;
  if (!aligned16(x) || !aligned16(w_router) || !aligned4(topk_ids) || !aligned4(topk_w) ||
      !aligned16(workspace))
    return MOE_FP4_ERR_MISALIGNED;
  if (workspace_bytes < moe_fp4_route_workspace_bytes(T, n_experts)) return MOE_FP4_ERR_WORKSPACE;
  if (T == 0) return MOE_FP4_OK;
  return from_hip(route_impl(x, w_router, T, hidden, n_experts, k, topk_ids, topk_w, workspace,
                             static_cast<hipStream_t>(stream)));
}

static bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

int moe_fp4_route_residual(const float* residual_in, const uint16_t* y_prev, float* residual_out,
                           uint16_t* x_out, float eps, const uint16_t* w_router, int T, int hidden,
                           int n_experts, int k, int32_t* topk_ids, float* topk_w, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!residual_in || !y_prev || !residual_out || !x_out || !w_router || !topk_ids || !topk_w ||
      !workspace)
    return MOE_FP4_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || !std::isfinite(eps)) return MOE_FP4_ERR_INVALID_ARG;
  int st = check_topk_args(T, n_experts, k);
  if (st != MOE_FP4_OK) return st;
  if (!valid_dim(hidden)) return MOE_FP4_ERR_BAD_SHAPE;
  if (!aligned16(residual_in) || !aligned16(y_prev) || !aligned16(residual_out) ||
      !aligned16(x_out) || !aligned16(w_router) || !aligned4(topk_ids) || !aligned4(topk_w) ||
      !aligned16(workspace))
    return MOE_FP4_ERR_MISALIGNED;
  if (workspace_bytes < moe_fp4_route_workspace_bytes(T, n_experts)) return MOE_FP4_ERR_WORKSPACE;
  // At T == 1 every router workgroup reads the whole of residual_in and y_prev while the
  // others write their slices of residual_out and x_out, so no output may overlap an input.
  const size_t rb = (size_t)T * (size_t)hidden * sizeof(float);
  const size_t xb = (size_t)T * (size_t)hidden * sizeof(uint16_t);
  if (ranges_overlap(residual_in, rb, residual_out, rb) || ranges_overlap(x_out, xb, y_prev, xb) ||
      ranges_overlap(x_out, xb, residual_in, rb) || ranges_overlap(residual_out, rb, y_prev, xb) ||
      ranges_overlap(x_out, xb, residual_out, rb))
    return MOE_FP4_ERR_INVALID_ARG;
  if (T == 0) return MOE_FP4_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* sync = static_cast<uint32_t*>(workspace);
  double* logits = reinterpret_cast<double*>(static_cast<uint8_t*>(workspace) + kRouteSyncBytes);
  if (T == 1 && (size_t)route_decode_sync_words(n_experts) * 4 <= kRouteSyncBytes)
    return from_hip(launch_route_decode_norm(residual_in, y_prev, residual_out, x_out, eps, w_router,
                                             hidden, n_experts, k, sync, logits, topk_ids, topk_w, s));
  if (launch_residual_rmsnorm(residual_in, y_prev, residual_out, x_out, T, hidden, eps, s) != hipSuccess)
    return MOE_FP4_ERR_HIP;
  return from_hip(route_impl(x_out, w_router, T, hidden, n_experts, k, topk_ids, topk_w, workspace, s));
}

int moe_fp4_route_status(const void* workspace, size_t workspace_bytes, int32_t* status,
                         void* stream) {
  if (!workspace || !status) return MOE_FP4_ERR_INVALID_ARG;
  if (!aligned16(workspace) || !aligned4(status)) return MOE_FP4_ERR_MISALIGNED;
  if (workspace_bytes < kRouteSyncBytes) return MOE_FP4_ERR_WORKSPACE;
  return from_hip(launch_route_status(static_cast<const uint32_t*>(workspace), status,
                                      static_cast<hipStream_t>(stream)));
}

int moe_fp4_route_reset(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return MOE_FP4_ERR_INVALID_ARG;
  if (!aligned16(workspace)) return MOE_FP4_ERR_MISALIGNED;
  if (workspace_bytes < kRouteSyncBytes) return MOE_FP4_ERR_WORKSPACE;
  return from_hip(launch_route_reset(static_cast<uint32_t*>(workspace), kRouteSyncBytes,
                                     static_cast<hipStream_t>(stream)));
}

int moe_fp4_debug_route_spin_limit(long long polls) {
  set_route_spin_limit(polls);
  return MOE_FP4_OK;
}

int moe_fp4_route_logits(const float* logits, int T, int n_experts, int k, int32_t* topk_ids,
                         float* topk_w, void* stream) {
  if (!logits || !topk_ids || !topk_w) return MOE_FP4_ERR_INVALID_ARG;
  int st = check_topk_args(T, n_experts, k);
  if (st != MOE_FP4_OK) return st;
  if (!aligned4(logits) || !aligned4(topk_ids) || !aligned4(topk_w)) return MOE_FP4_ERR_MISALIGNED;
  if (T == 0) return MOE_FP4_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip((launch_topk_f32(logits, T, n_experts, k, topk_ids, topk_w, s)));
}

// Token count from which the automatic path choice takes the grouped GEMM path.
constexpr int kGroupedMinTokens = 24;

size_t moe_fp4_workspace_bytes(int T, int k, int n_experts, int hidden, int inter) {
  if (T < 0 || k < 1 || k > kMaxK || n_experts <= 0 || !valid_dim(hidden) || !valid_dim(inter))
    return 0;
  if (T == 0) return 0;
  // decode path: h for every (token, slot) pair, bf16; grouped path: see batched_layout
  const size_t decode = align256((size_t)T * (size_t)k * (size_t)inter * 2);
  const size_t grouped = batched_layout(T, k, n_experts, hidden, inter).bytes;
  return std::max(std::max(decode, grouped), small_m_workspace_bytes(T, k, hidden, inter));
}

static bool lds_fits(int k, int inter) { return (size_t)k * (size_t)inter * 2 <= (size_t)kMaxLdsH; }

// The FFN on a workspace of moe_fp4_workspace_bytes; path already validated.
static hipError_t ffn_impl(const uint16_t* x, const int32_t* topk_ids, const float* topk_w, int T,
                           int k, const uint8_t* pk, int n_experts, int hidden, int inter,
                           uint16_t* y, void* workspace, int path, hipStream_t s) {
  if (path == MOE_FP4_PATH_GROUPED || path == MOE_FP4_PATH_GROUPED_FP8)
    return launch_batched_ffn(x, topk_ids, topk_w, T, k, pk, n_experts, hidden, inter, y,
                              workspace, path == MOE_FP4_PATH_GROUPED ? 2 : 1, s);
  if (path == MOE_FP4_PATH_SMALL_M)
    return launch_small_m_ffn(x, topk_ids, topk_w, T, k, pk, n_experts, hidden, inter, workspace,
                              y, s);
  uint16_t* hbuf = static_cast<uint16_t*>(workspace);
  hipError_t e = launch_gate_up(x, topk_ids, T, k, pk, n_experts, hidden, inter, hbuf, s);
  if (e != hipSuccess) return e;
  return launch_down_combine(topk_ids, topk_w, T, k, pk, n_experts, hidden, inter, hbuf, y, s);
}

// Resolves MOE_FP4_PATH_AUTO and checks the shape limits of the chosen path.
static bool small_m_fits(int T, int k, int hidden, int inter) {
  return T >= 2 && (long)T * k <= 256 && small_m_rows(T, hidden, inter) >= 2;
}

static int choose_path(int path, int T, int k, int n_experts, int hidden, int inter) {
  if (path == MOE_FP4_PATH_AUTO) {
    if (T >= kGroupedMinTokens && n_experts <= kMaxExpertsTopk)
      path = MOE_FP4_PATH_GROUPED;
    else if (small_m_fits(T, k, hidden, inter))
      path = MOE_FP4_PATH_SMALL_M;
    else
      path = MOE_FP4_PATH_DECODE;
    if (path == MOE_FP4_PATH_DECODE && !lds_fits(k, inter) && n_experts <= kMaxExpertsTopk)
      path = MOE_FP4_PATH_GROUPED;
  }
  if (path == MOE_FP4_PATH_DECODE) return lds_fits(k, inter) ? path : MOE_FP4_ERR_BAD_SHAPE;
  if (path == MOE_FP4_PATH_GROUPED || path == MOE_FP4_PATH_GROUPED_FP8)
    return n_experts <= kMaxExpertsTopk ? path : MOE_FP4_ERR_BAD_SHAPE;
  if (path == MOE_FP4_PATH_SMALL_M)
    return (T == 0 || small_m_fits(T, k, hidden, inter)) ? path : MOE_FP4_ERR_BAD_SHAPE;
  return MOE_FP4_ERR_INVALID_ARG;
}

int moe_fp4_expert_ffn_ex(const uint16_t* x, const int32_t* topk_ids, const float* topk_w, int T,
                          int k, const void* packed, int n_experts, int hidden, int inter,
                          uint16_t* y, void* workspace, size_t workspace_bytes, int path,
                          void* stream) {
  if (!x || !topk_ids || !topk_w || !packed || !y || !workspace) return MOE_FP4_ERR_INVALID_ARG;
  if (T < 0 || n_experts <= 0 || k < 1 || k > kMaxK || k > n_experts) return MOE_FP4_ERR_INVALID_ARG;
  if (!valid_dim(hidden) || !valid_dim(inter)) return MOE_FP4_ERR_BAD_SHAPE;
  const int chosen = choose_path(path, T, k, n_experts, hidden, inter);
  if (chosen < 0) return chosen;
  if (!aligned16(x) || !aligned4(topk_ids) || !aligned4(topk_w) || !aligned16(packed) ||
      !aligned16(y) || !aligned16(workspace))
    return MOE_FP4_ERR_MISALIGNED;
  if (workspace_bytes < moe_fp4_workspace_bytes(T, k, n_experts, hidden, inter))
    return MOE_FP4_ERR_WORKSPACE;
  if (T == 0) return MOE_FP4_OK;
  return from_hip(ffn_impl(x, topk_ids, topk_w, T, k, static_cast<const uint8_t*>(packed),
                           n_experts, hidden, inter, y, workspace, chosen,
                           static_cast<hipStream_t>(stream)));
}

int moe_fp4_expert_ffn(const uint16_t* x, const int32_t* topk_ids, const float* topk_w, int T,
                       int k, const void* packed, int n_experts, int hidden, int inter,
                       uint16_t* y, void* workspace, size_t workspace_bytes, void* stream) {
  return moe_fp4_expert_ffn_ex(x, topk_ids, topk_w, T, k, packed, n_experts, hidden, inter, y,
                               workspace, workspace_bytes, MOE_FP4_PATH_AUTO, stream);
}

size_t moe_fp4_moe_forward_workspace_bytes(int T, int k, int n_experts, int hidden, int inter) {
  if (T < 0 || n_experts <= 0) return 0;
  const size_t ffn = moe_fp4_workspace_bytes(T, k, n_experts, hidden, inter);
  if (ffn == 0) return 0;
  return moe_fp4_route_workspace_bytes(T, n_experts) + ffn;
}

int moe_fp4_moe_forward(const uint16_t* x, const uint16_t* w_router, int T, int hidden,
                        int n_experts, int k, const void* packed, int inter, int32_t* topk_ids,
                        float* topk_w, uint16_t* y, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (!x || !w_router || !packed || !topk_ids || !topk_w || !y || !workspace)
    return MOE_FP4_ERR_INVALID_ARG;
  int st = check_topk_args(T, n_experts, k);
  if (st != MOE_FP4_OK) return st;
  if (!valid_dim(hidden) || !valid_dim(inter)) return MOE_FP4_ERR_BAD_SHAPE;
  const int chosen = choose_path(MOE_FP4_PATH_AUTO, T, k, n_experts, hidden, inter);
  if (chosen < 0) return chosen;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(packed) || !aligned4(topk_ids) ||
      !aligned4(topk_w) || !aligned16(y) || !aligned16(workspace))
    return MOE_FP4_ERR_MISALIGNED;
  if (workspace_bytes < moe_fp4_moe_forward_workspace_bytes(T, k, n_experts, hidden, inter))
    return MOE_FP4_ERR_WORKSPACE;
  if (T == 0) return MOE_FP4_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (route_impl(x, w_router, T, hidden, n_experts, k, topk_ids, topk_w, workspace, s) != hipSuccess)
    return MOE_FP4_ERR_HIP;
  void* ffn_ws = static_cast<uint8_t*>(workspace) + moe_fp4_route_workspace_bytes(T, n_experts);
  return from_hip(ffn_impl(x, topk_ids, topk_w, T, k, static_cast<const uint8_t*>(packed),
                           n_experts, hidden, inter, y, ffn_ws, chosen, s));
}

// ---------------------------------------------------------------------------------------
// The no-allocation variant of moe_fp4_moe_forward: its workspace is this file-scope device
// array (each GPU the library runs on holds its own copy until the process ends). In host
// code `scratch` names a host-side stand-in, not the device memory, so host code uses only
// the per-device address that hipGetSymbolAddress returns, taken once per device on the
// entry point's first call there (with that device current) and kept here.
// ---------------------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = MOE_FP4_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of `scratch` (nullptr when the device or the call fails).
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

int moe_fp4_moe_forward_noalloc(const uint16_t* x, const uint16_t* w_router, int T, int hidden,
                                int n_experts, int k, const void* packed, int inter,
                                int32_t* topk_ids, float* topk_w, uint16_t* y, void* stream) {
  if (!x || !w_router || !packed || !topk_ids || !topk_w || !y) return MOE_FP4_ERR_INVALID_ARG;
  int st = check_topk_args(T, n_experts, k);
  if (st != MOE_FP4_OK) return st;
  if (!valid_dim(hidden) || !valid_dim(inter)) return MOE_FP4_ERR_BAD_SHAPE;
  if (choose_path(MOE_FP4_PATH_AUTO, T, k, n_experts, hidden, inter) < 0) return MOE_FP4_ERR_BAD_SHAPE;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(packed) || !aligned4(topk_ids) ||
      !aligned4(topk_w) || !aligned16(y))
    return MOE_FP4_ERR_MISALIGNED;
  if (T == 0) return MOE_FP4_OK;
  const size_t need = moe_fp4_moe_forward_workspace_bytes(T, k, n_experts, hidden, inter);
  if (need == 0 || need > kNoAllocScratchBytes) return MOE_FP4_ERR_TOO_LARGE;
  void* ws = scratch_address();
  if (!ws) return MOE_FP4_ERR_HIP;
  return moe_fp4_moe_forward(x, w_router, T, hidden, n_experts, k, packed, inter, topk_ids, topk_w,
                             y, ws, kNoAllocScratchBytes, stream);
}

int moe_fp4_residual_init(const uint16_t* x, float* residual, int T, int hidden, void* stream) {
  if (!x || !residual || T < 0 || hidden <= 0) return MOE_FP4_ERR_INVALID_ARG;
  if (!aligned4(residual) || (reinterpret_cast<uintptr_t>(x) & 1u)) return MOE_FP4_ERR_MISALIGNED;
  if (T == 0) return MOE_FP4_OK;
  return from_hip(launch_residual_init(x, residual, T, hidden, static_cast<hipStream_t>(stream)));
}

int moe_fp4_residual_rmsnorm(float* residual, const uint16_t* y, uint16_t* x_out, int T,
                             int hidden, float eps, void* stream) {
  if (!residual || !y || !x_out || T < 0 || hidden <= 0 || !(eps >= 0.f)) return MOE_FP4_ERR_INVALID_ARG;
  if (hidden % 8 != 0 || hidden > kMaxDim) return MOE_FP4_ERR_BAD_SHAPE;
  if (!aligned16(residual) || !aligned16(y) || !aligned16(x_out)) return MOE_FP4_ERR_MISALIGNED;
  if (T == 0) return MOE_FP4_OK;
  return from_hip(launch_residual_rmsnorm(residual, y, residual, x_out, T, hidden, eps,
                                          static_cast<hipStream_t>(stream)));
}

int moe_fp4_prefetch_experts(const int32_t* ids, int n_ids, const void* packed, int n_experts,
                             int hidden, int inter, int matrices, uint32_t* sink, void* stream) {
  if (!ids || !packed || !sink || n_ids < 0 || n_experts <= 0) return MOE_FP4_ERR_INVALID_ARG;
  if (matrices < 1 || matrices > 7) return MOE_FP4_ERR_INVALID_ARG;
  if (n_ids > (1 << 16)) return MOE_FP4_ERR_INVALID_ARG;
  if (!valid_dim(hidden) || !valid_dim(inter)) return MOE_FP4_ERR_BAD_SHAPE;
  if (!aligned4(ids) || !aligned16(packed) || !aligned4(sink)) return MOE_FP4_ERR_MISALIGNED;
  if (n_ids == 0) return MOE_FP4_OK;
  return from_hip(launch_prefetch_experts(ids, n_ids, static_cast<const uint8_t*>(packed), n_experts,
                                          hidden, inter, matrices, sink,
                                          static_cast<hipStream_t>(stream)));
}

int moe_fp4_validate_ids(const int32_t* topk_ids, int T, int k, int n_experts, int32_t* bad_count,
                         void* stream) {
  if (!topk_ids || !bad_count || T < 0 || k < 1 || n_experts <= 0) return MOE_FP4_ERR_INVALID_ARG;
  if (!aligned4(topk_ids)) return MOE_FP4_ERR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(launch_validate_ids(topk_ids, T, k, n_experts, bad_count, s));
}

int moe_fp4_debug_dequant(const void* packed, int n_experts, int hidden, int inter, int expert,
                          int matrix, float* out, void* stream) {
  if (!packed || !out || n_experts <= 0) return MOE_FP4_ERR_INVALID_ARG;
  if (expert < 0 || expert >= n_experts || matrix < 0 || matrix > 2) return MOE_FP4_ERR_INVALID_ARG;
  if (!valid_dim(hidden) || !valid_dim(inter)) return MOE_FP4_ERR_BAD_SHAPE;
  if (!aligned16(packed) || !aligned16(out)) return MOE_FP4_ERR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(launch_debug_dequant(static_cast<const uint8_t*>(packed), hidden, inter, expert,
                                       matrix, out, s));
}

size_t moe_fp4_fp8_packed_bytes(int rows, int cols) {
  if (!valid_dim(rows) || !valid_dim(cols)) return 0;
  return fp8_packed_bytes(rows, cols);
}

int moe_fp4_fp8_pack(const uint8_t* codes, const float* scale_inv, int rows, int cols, void* packed,
                     size_t packed_bytes, void* stream) {
  if (!codes || !scale_inv || !packed) return MOE_FP4_ERR_INVALID_ARG;
  if (!valid_dim(rows) || !valid_dim(cols)) return MOE_FP4_ERR_BAD_SHAPE;
  if (!aligned16(codes) || !aligned4(scale_inv) || !aligned16(packed)) return MOE_FP4_ERR_MISALIGNED;
  if (packed_bytes < fp8_packed_bytes(rows, cols)) return MOE_FP4_ERR_WORKSPACE;
  return from_hip(launch_fp8_pack(codes, scale_inv, rows, cols, static_cast<uint8_t*>(packed),
                                  static_cast<hipStream_t>(stream)));
}

int moe_fp4_fp8_linear(const uint16_t* x, int T, const void* packed, int rows, int cols,
                       uint16_t* y, void* stream) {
  if (!x || !packed || !y || T < 0) return MOE_FP4_ERR_INVALID_ARG;
  if (!valid_dim(rows) || !valid_dim(cols)) return MOE_FP4_ERR_BAD_SHAPE;
  if (!aligned16(x) || !aligned16(packed) || !aligned16(y)) return MOE_FP4_ERR_MISALIGNED;
  if (T == 0) return MOE_FP4_OK;
  return from_hip(launch_fp8_linear(x, T, static_cast<const uint8_t*>(packed), rows, cols, y,
                                    static_cast<hipStream_t>(stream)));
}

int moe_fp4_fp8_swiglu(const uint16_t* x, int T, const void* gate, const void* up, int inter,
                       int hidden, uint16_t* h, void* stream) {
  if (!x || !gate || !up || !h || T < 0) return MOE_FP4_ERR_INVALID_ARG;
  if (!valid_dim(inter) || !valid_dim(hidden)) return MOE_FP4_ERR_BAD_SHAPE;
  if (!aligned16(x) || !aligned16(gate) || !aligned16(up) || !aligned16(h)) return MOE_FP4_ERR_MISALIGNED;
  if (T == 0) return MOE_FP4_OK;
  return from_hip(launch_fp8_swiglu(x, T, static_cast<const uint8_t*>(gate),
                                    static_cast<const uint8_t*>(up), inter, hidden, h,
                                    static_cast<hipStream_t>(stream)));
}

size_t moe_fp4_shared_expert_workspace_bytes(int T, int inter) {
  if (T < 0 || !valid_dim(inter)) return 0;
  return align256((size_t)T * (size_t)inter * 2);
}

int moe_fp4_shared_expert(const uint16_t* x, int T, const void* gate, const void* up,
                          const void* down, int hidden, int inter, uint16_t* y, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!x || !gate || !up || !down || !y || !workspace || T < 0) return MOE_FP4_ERR_INVALID_ARG;
  if (!valid_dim(inter) || !valid_dim(hidden)) return MOE_FP4_ERR_BAD_SHAPE;
  if (!aligned16(x) || !aligned16(gate) || !aligned16(up) || !aligned16(down) || !aligned16(y) ||
      !aligned16(workspace))
    return MOE_FP4_ERR_MISALIGNED;
  if (workspace_bytes < moe_fp4_shared_expert_workspace_bytes(T, inter)) return MOE_FP4_ERR_WORKSPACE;
  if (T == 0) return MOE_FP4_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* h = static_cast<uint16_t*>(workspace);
  hipError_t e = launch_fp8_swiglu(x, T, static_cast<const uint8_t*>(gate),
                                   static_cast<const uint8_t*>(up), inter, hidden, h, s);
  if (e != hipSuccess) return from_hip(e);
  return from_hip(launch_fp8_linear(h, T, static_cast<const uint8_t*>(down), hidden, inter, y, s));
}

size_t moe_fp4_debug_act_quant_bytes(int T, int hidden) {
  if (T < 0 || !valid_dim(hidden)) return 0;
  return debug_act_quant_bytes(T, hidden);
}

int moe_fp4_debug_act_quant(const uint16_t* x, int T, int hidden, int terms, void* workspace,
                            size_t workspace_bytes, float* out, void* stream) {
  if (!x || !out || !workspace || T < 0 || terms < 1 || terms > 2) return MOE_FP4_ERR_INVALID_ARG;
  if (!valid_dim(hidden)) return MOE_FP4_ERR_BAD_SHAPE;
  if (!aligned16(x) || !aligned16(out) || !aligned16(workspace)) return MOE_FP4_ERR_MISALIGNED;
  if (workspace_bytes < debug_act_quant_bytes(T, hidden)) return MOE_FP4_ERR_WORKSPACE;
  if (T == 0) return MOE_FP4_OK;
  return from_hip(launch_debug_act_quant(x, T, hidden, terms, workspace, out,
                                         static_cast<hipStream_t>(stream)));
}

int moe_fp4_debug_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0) return MOE_FP4_ERR_INVALID_ARG;
  if (!aligned16(src) || !aligned4(sink)) return MOE_FP4_ERR_MISALIGNED;
  return from_hip(launch_probe_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream)));
}

int moe_fp4_debug_mfma_loop(int fmt_a, int n_workgroups, int iters, uint32_t* sink,
                            void* stream) {
  static_assert(MOE_FP4_PROBE_MFMA_CHAINS > 0, "chains");
  if (!sink || (fmt_a != 0 && fmt_a != 4)) return MOE_FP4_ERR_INVALID_ARG;
  if (n_workgroups < 1 || n_workgroups > (1 << 20) || iters < 1 || iters > (1 << 20))
    return MOE_FP4_ERR_INVALID_ARG;
  if (!aligned4(sink)) return MOE_FP4_ERR_MISALIGNED;
  if (probe_mfma_chains() != MOE_FP4_PROBE_MFMA_CHAINS) return MOE_FP4_ERR_INVALID_ARG;
  return from_hip(launch_probe_mfma_loop(fmt_a, n_workgroups, iters, sink,
                                         static_cast<hipStream_t>(stream)));
}

int moe_fp4_timing_enable(int enable) {
  timing().enabled = enable != 0;
  return MOE_FP4_OK;
}

int moe_fp4_timing_reset(void) {
  TimingState& st = timing();
  for (auto& r : st.recs) {
    st.free_events.push_back(r.start);
    st.free_events.push_back(r.stop);
  }
  st.recs.clear();
  return MOE_FP4_OK;
}

int moe_fp4_timing_read(int kind, int* launches, double* total_ms) {
  if (!launches || !total_ms || kind < 0 || kind >= MOE_FP4_KERNEL_KINDS) return MOE_FP4_ERR_INVALID_ARG;
  TimingState& st = timing();
  int n = 0;
  double sum = 0.0;
  for (auto& r : st.recs) {
    if (r.kind != kind) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return MOE_FP4_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return MOE_FP4_ERR_HIP;
    sum += ms;
    ++n;
  }
  *launches = n;
  *total_ms = sum;
  return MOE_FP4_OK;
}

}  // extern "C"
