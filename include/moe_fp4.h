/*
 * moe_fp4.h -- C ABI of the routed FP4 expert FFN library for AMD MI355X (gfx950).
 *
 * The operation is the routed-expert FFN of a DeepSeek-style MoE decoder layer: every
 * token picks k of E SwiGLU experts; each expert holds three FP4 E2M1 matrices with one
 * ue8m0 power-of-two scale per 32 elements along K; the token's output is the
 * router-weighted sum of its experts' outputs.
 *
 * Pages this follows (cited by title and section):
 *  [A100-FP4] shi3z, "DeepSeek v4.1 Flashを動かしたくてFP4に対応していないA100を、33tok/sから
 *             673 tok/sまで持っていって気がつくと公式APIより速くなっていた話" (note.com) and its
 *             Chinese translation "把不支持 FP4 的 A100 拉到 673 tok/s".
 *  [8GB-GPU]  "在 8 GB 显卡上运行 510 GB 的 DeepSeek-V4.1-Flash——以及三个从不抛错的 Bug".
 *
 * Conventions for every call:
 *  - All array arguments are DEVICE pointers (hipMalloc'd or equivalent) unless stated.
 *    The caller allocates and owns every buffer; no call allocates device memory, and
 *    apart from the static scratch array of moe_fp4_moe_forward_noalloc (part of the
 *    library's code object, MOE_FP4_NOALLOC_SCRATCH_BYTES per GPU) the library keeps no
 *    state between calls.
 *  - bfloat16 values are passed as uint16_t bit patterns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). Every call
 *    only enqueues work on that stream and returns; none synchronises with the host, so
 *    routing ids never travel to the host ([8GB-GPU], section 提速之路：v1 到 v4: the
 *    per-expert host synchronisation on indices was a measured cost).
 *  - Return value: MOE_FP4_OK (0) or a negative status below. Arguments are checked on the
 *    host before anything is enqueued; a non-OK status means nothing was enqueued.
 *    Faults inside a kernel surface at the caller's next synchronisation.
 *  - T = 0 (no tokens) is a no-op that returns MOE_FP4_OK.
 *  - Shapes: hidden and inter must be positive multiples of 32 and at most 16384;
 *    1 <= k <= min(n_experts, 8); the decode FFN path needs k * inter <= 32768 (the k h
 *    vectors of a token are staged in 64 KB of LDS), the grouped path n_experts <= 2048.
 *  - Alignment: topk_ids, topk_w and the fp32 logits of moe_fp4_route_logits must be
 *    4-byte aligned (so a row slice of a [T x k] array can be passed); every other device
 *    pointer (activations, weights, packed experts, outputs, workspaces) 16-byte aligned.
 */
#ifndef MOE_FP4_H
#define MOE_FP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_FP4_OK 0
#define MOE_FP4_ERR_INVALID_ARG (-1)   /* null pointer, negative size, k out of range */
#define MOE_FP4_ERR_BAD_SHAPE (-2)     /* hidden or inter not a multiple of 32 / too large */
#define MOE_FP4_ERR_MISALIGNED (-3)    /* a device pointer breaks the alignment rule above */
#define MOE_FP4_ERR_WORKSPACE (-4)     /* workspace or packed buffer smaller than required */
#define MOE_FP4_ERR_HIP (-5)           /* a HIP launch or runtime call failed */
#define MOE_FP4_ERR_TOO_LARGE (-6)     /* needs more than the no-allocation entry point's scratch */

/* Library version, major * 10000 + minor * 100 + patch. */
int moe_fp4_version(void);

/* Human-readable text for a status code (static storage, never NULL). */
const char* moe_fp4_strerror(int status);

/* ------------------------------------------------------------------------------------
 * Expert weights: canonical blob and packed device layout.
 *
 * Canonical blob of one expert ([8GB-GPU], section 方案：不重写模型，只迁移其存储: the three
 * matrices of an expert lie next to each other, the scales are a separate block;
 * section 每 token 字节数决定一切: 17.93 MiB per expert at hidden 4096, inter 2880):
 *   codes : gate [inter x hidden/2] | up [inter x hidden/2] | down [hidden x inter/2]
 *           uint8, row-major [out x in]; a byte holds two E2M1 codes, the low nibble is
 *           the even K index. E2M1: bit 3 sign, bits 2:1 exponent (bias 1), bit 0
 *           mantissa ([A100-FP4], section 「FP4非対応」という言葉を疑う).
 *   scales: gate [inter x hidden/32] | up [inter x hidden/32] | down [hidden x inter/32]
 *           uint8 ue8m0: byte e scales its 32-element K block by 2^(e-127); e = 255 is NaN.
 * For n_experts experts the canonical arrays are codes [E][3*hidden*inter/2] and
 * scales [E][3*hidden*inter/32], expert after expert.
 * ------------------------------------------------------------------------------------ */

/* Bytes of the packed device layout for n_experts experts (0 if the shape is invalid). */
size_t moe_fp4_packed_bytes(int n_experts, int hidden, int inter);

/* Byte distance between consecutive experts in the packed layout (a multiple of 256), so
 * that a caller can pack a large expert set one expert (or one chunk) at a time by passing
 * packed + e * stride. 0 if the shape is invalid. */
size_t moe_fp4_packed_expert_stride(int hidden, int inter);

/* Load-time re-layout ([A100-FP4], section 但 CPU 也没那么快: weights are rearranged once at
 * load time into the order the compute kernels read best).
 * codes, scales: canonical arrays for n_experts experts (device).
 * packed: destination of at least moe_fp4_packed_bytes(n_experts, hidden, inter) bytes.
 * Errors: INVALID_ARG, BAD_SHAPE, MISALIGNED, WORKSPACE (packed_bytes too small), HIP. */
int moe_fp4_pack(const uint8_t* codes, const uint8_t* scales, int n_experts, int hidden,
                 int inter, void* packed, size_t packed_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * Routing ([8GB-GPU], section 每 token 字节数决定一切: 6 of 384 experts per token).
 * logits[t, e] = sum_h w_router[e, h] * x[t, h], accumulated in fp64; the k largest
 * logits of each token are returned in descending order, equal logits ordered by
 * ascending expert id; topk_w[t, j] = softmax over the token's k selected logits
 * (equivalently the full softmax renormalised over the selection).
 * ------------------------------------------------------------------------------------ */

/* Workspace bytes moe_fp4_route needs for T tokens and n_experts experts. */
size_t moe_fp4_route_workspace_bytes(int T, int n_experts);

/* x [T x hidden] bf16, w_router [n_experts x hidden] bf16 (row-major), outputs
 * topk_ids int32 [T x k], topk_w fp32 [T x k]. workspace: device scratch of at least
 * moe_fp4_route_workspace_bytes(T, n_experts) bytes, owned by the caller. Its first 16 KB
 * hold synchronisation words that a batch-1 call (T == 1: GEMV and selection in one
 * launch) carries from call to call; their initial contents do not matter, the caller
 * must not write them between calls, and calls that may run concurrently need distinct
 * workspaces. The rest is scratch whose contents on entry are ignored.
 * Errors: INVALID_ARG, BAD_SHAPE, MISALIGNED, WORKSPACE, HIP. */
int moe_fp4_route(const uint16_t* x, const uint16_t* w_router, int T, int hidden, int n_experts,
                  int k, int32_t* topk_ids, float* topk_w, void* workspace,
                  size_t workspace_bytes, void* stream);

/* A batch-1 call waits, boundedly, for the router logits its other workgroups publish in
 * the synchronisation area (about a second of polling; only a GPU that cannot run all of
 * the call's workgroups meanwhile reaches the bound). If the bound is reached the call
 * gives up: it writes topk_ids = -1 and topk_w = 0 (ids every FFN path skips and
 * moe_fp4_validate_ids counts) and marks the area as failed. Workgroups that start after
 * the give-up can leave records a later call would take for its own, so the mark is
 * sticky: every later batch-1 call on that workspace (moe_fp4_route, moe_fp4_route_residual,
 * moe_fp4_moe_forward) writes -1 / 0 as well until moe_fp4_route_reset clears the area.
 * moe_fp4_route_status writes 1 to the device int32 *status if the area of `workspace`
 * (the route or moe_fp4_moe_forward workspace, at least 16 KB) holds the mark, else 0.
 * moe_fp4_route_reset zeroes the 16 KB area with a fill kernel on `stream` (no memset node,
 * so it can be captured in a graph); the next call starts afresh. Both are stream-ordered.
 * Errors: INVALID_ARG (null), MISALIGNED (workspace 16-byte, status 4-byte), WORKSPACE
 * (workspace_bytes < 16384), HIP. */
int moe_fp4_route_status(const void* workspace, size_t workspace_bytes, int32_t* status,
                         void* stream);
int moe_fp4_route_reset(void* workspace, size_t workspace_bytes, void* stream);

/* Debug helper for tests of the give-up above: sets the number of polls per logit record
 * after which later batch-1 route launches give up (0: at once, without polling; negative:
 * the default bound). A host-side setting of this process, read at each launch; not
 * thread-safe. */
int moe_fp4_debug_route_spin_limit(long long polls);

/* The selection and weighting of moe_fp4_route applied to given fp32 logits
 * [T x n_experts] (for workloads whose router logits are drawn directly). No workspace. */
int moe_fp4_route_logits(const float* logits, int T, int n_experts, int k, int32_t* topk_ids,
                         float* topk_w, void* stream);

/* ------------------------------------------------------------------------------------
 * Routed expert FFN with the router-weighted combine.
 * For every token t and slot j with e = topk_ids[t, j] in [0, n_experts):
 *   g = W_gate[e] x_t, u = W_up[e] x_t, h = silu(g) * u, y_e = W_down[e] h,
 * and y[t] = sum_j topk_w[t, j] * y_e, summed in ascending expert id (so permuting a
 * token's (id, weight) pairs does not change the result). Ids outside [0, n_experts)
 * contribute nothing; duplicate ids add up; weights are used as given.
 * The pages state the problem this way: per token, 6 of 384 experts, each an FP4 blob of
 * three adjacent matrices with a separate ue8m0 scale block, read and applied per token
 * ([8GB-GPU], sections 每 token 字节数决定一切 and 方案：不重写模型，只迁移其存储); the FP4 codes
 * meet the matrix cores without being expanded in memory ([A100-FP4], section
 * 「FP4非対応」という言葉を疑う).
 * Numerics: FP4 weights are dequantised exactly in registers, products and sums are fp32,
 * h is rounded to bf16 before the down projection, y is rounded to bf16. Every ue8m0 byte is
 * applied exactly (255 = NaN, which propagates to the outputs it reaches); a dequantised
 * weight of magnitude 2^128 or more (byte 253 with |E2M1| >= 4, byte 254 with |E2M1| >= 2)
 * is outside the bf16 operand range of the decode and small-M paths and becomes +-inf there.
 * ------------------------------------------------------------------------------------ */

/* Workspace bytes moe_fp4_expert_ffn (any path) needs: the larger of h of every (token,
 * slot) pair in bf16 (decode path) and the grouped path's sort tables, MX activations
 * and per-pair fp32 outputs (about T * k * (hidden * 4 + 2 * inter) bytes). 0 for invalid
 * arguments. */
size_t moe_fp4_workspace_bytes(int T, int k, int n_experts, int hidden, int inter);

/* x [T x hidden] bf16; topk_ids int32 [T x k]; topk_w fp32 [T x k];
 * packed: the output of moe_fp4_pack for n_experts experts; y [T x hidden] bf16 (output,
 * may not alias x); workspace of at least moe_fp4_workspace_bytes(...) bytes, owned by the
 * caller, contents on entry ignored; calls that may run concurrently need distinct
 * workspaces.
 * Errors: INVALID_ARG, BAD_SHAPE, MISALIGNED, WORKSPACE, HIP. */
int moe_fp4_expert_ffn(const uint16_t* x, const int32_t* topk_ids, const float* topk_w, int T,
                       int k, const void* packed, int n_experts, int hidden, int inter,
                       uint16_t* y, void* workspace, size_t workspace_bytes, void* stream);

/* The same operation with an explicit choice of kernels ([A100-FP4], section
 * 批处理不是「同时处理几个人」: tokens routed to the same expert can share one read of its
 * weights, and weight reads are the cost that matters in an MoE layer).
 *  MOE_FP4_PATH_DECODE: every (token, slot) pair streams its expert's weights (two
 *    launches; best at batch 1; needs k * inter <= 32768).
 *  MOE_FP4_PATH_GROUPED: pairs are grouped by expert on the device (no host readback) and
 *    run through a grouped GEMM on the block-scaled FP4 matrix cores; the activations x and
 *    h enter the matrix cores as two-term MXFP6 (E2M3 hi + lo, one ue8m0 scale per 32
 *    elements each; E2M3 operands run at the FP4 rate), accumulation is fp32, each pair's
 *    weighted output is combined per token in canonical slot order (five launches; needs
 *    n_experts <= 2048). A NaN or infinity in a 32-element block of x or h (E2M3 has
 *    neither) gives the block a NaN scale, so the outputs it reaches are NaN.
 *  MOE_FP4_PATH_SMALL_M: for a few tokens per call (several draft tokens of one sequence,
 *    a few streams): the pairs that chose the same expert share one read of its weights in
 *    groups of up to G pairs (the tokens of a group are rows of one matrix-core tile), h is
 *    bit-identical to DECODE's, each pair's weighted output is combined per token in
 *    canonical slot order (three launches). G is the largest power of two <= min(T, 8)
 *    with G * max(hidden, inter) <= 16384 (the group's bf16 rows fit in 32 KB of LDS);
 *    needs 2 <= T, T * k <= 256 and G >= 2 (max(hidden, inter) <= 8192).
 *  MOE_FP4_PATH_GROUPED_FP8: opt-in; GROUPED with the activations x and h as one MXFP8
 *    term (E4M3, one ue8m0 scale per 32 elements): DeepSeek's FP8 activation numerics
 *    ([8GB-GPU], section RTX 50xx 上的三个从不抛错的 Bug: activations quantised with ue8m0
 *    scales). Two thirds of GROUPED's activation bytes and the same matrix-core time (one
 *    FP8 product instead of two at the FP4 rate); the result is that of the quantised
 *    activations, which on the 384-expert layer lies further from the exact
 *    bf16 computation than the 2e-2 normwise bar of the other paths. AUTO never picks it.
 *  MOE_FP4_PATH_AUTO: GROUPED from 24 tokens on; SMALL_M from 2 to 23 tokens where its
 *    limits hold; DECODE otherwise (one token, or a shape SMALL_M refuses). Measured on the
 *    384-expert layer: SMALL_M is faster than DECODE at every T >= 2, with uniform and with
 *    correlated routing; GROUPED overtakes SMALL_M between 12 and 24 tokens when the tokens
 *    share most experts, and not below 42 tokens with uniform routing.
 * moe_fp4_expert_ffn is this call with MOE_FP4_PATH_AUTO. The workspace size covers every
 * path. Errors: as moe_fp4_expert_ffn; an unknown path is INVALID_ARG, a shape the chosen
 * path cannot take is BAD_SHAPE. */
#define MOE_FP4_PATH_AUTO 0
#define MOE_FP4_PATH_DECODE 1
#define MOE_FP4_PATH_GROUPED 2
#define MOE_FP4_PATH_SMALL_M 3
#define MOE_FP4_PATH_GROUPED_FP8 4
int moe_fp4_expert_ffn_ex(const uint16_t* x, const int32_t* topk_ids, const float* topk_w, int T,
                          int k, const void* packed, int n_experts, int hidden, int inter,
                          uint16_t* y, void* workspace, size_t workspace_bytes, int path,
                          void* stream);

/* ------------------------------------------------------------------------------------
 * Whole routed-expert layer in one call: moe_fp4_route followed by moe_fp4_expert_ffn on
 * one workspace (three kernel launches for a batch-1 call: router GEMV with selection,
 * gate/up/SiLU, down + combine). Same results as the two calls in sequence: topk_ids /
 * topk_w receive the routing (bit-identical to moe_fp4_route), y the layer output
 * (bit-identical to moe_fp4_expert_ffn). Cutting launches per layer is the pages' own
 * lesson ([A100-FP4], section 然后又发现每 token 启动 2000 次内核). The workspace's first
 * 16 KB follow the rules given for moe_fp4_route.
 * ------------------------------------------------------------------------------------ */

/* Workspace bytes moe_fp4_moe_forward needs. */
size_t moe_fp4_moe_forward_workspace_bytes(int T, int k, int n_experts, int hidden, int inter);

/* x [T x hidden] bf16; w_router [n_experts x hidden] bf16; packed: moe_fp4_pack output;
 * outputs topk_ids int32 [T x k], topk_w fp32 [T x k], y [T x hidden] bf16.
 * Errors: INVALID_ARG, BAD_SHAPE, MISALIGNED, WORKSPACE, HIP. */
int moe_fp4_moe_forward(const uint16_t* x, const uint16_t* w_router, int T, int hidden,
                        int n_experts, int k, const void* packed, int inter, int32_t* topk_ids,
                        float* topk_w, uint16_t* y, void* workspace, size_t workspace_bytes,
                        void* stream);

/* For callers that cannot allocate device memory (code under stream or graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): moe_fp4_moe_forward with no
 * workspace argument. Its workspace is a static device array of
 * MOE_FP4_NOALLOC_SCRATCH_BYTES bytes inside the library; every GPU the call runs on holds
 * its own copy from the first call there until the process ends. The call allocates
 * nothing (no hipMalloc, no allocating library routine); the caller still owns x, the
 * router, the packed experts and the outputs, under the rules of moe_fp4_moe_forward, and
 * gets the same results (the same kernels on the same workspace layout).
 * The limit: moe_fp4_moe_forward_workspace_bytes(T, k, n_experts, hidden, inter) must not
 * exceed MOE_FP4_NOALLOC_SCRATCH_BYTES, else MOE_FP4_ERR_TOO_LARGE and nothing is enqueued
 * (at hidden 4096, inter 2880, 384 experts, top-6: up to 114 tokens per call).
 * All calls on one GPU share that GPU's array, which keeps the last call's state (the
 * route's synchronisation words carry from call to call as in moe_fp4_route): calls that
 * may overlap on one GPU (different streams, different host threads) race and must be
 * serialised by the caller. A batch-1 route give-up (see moe_fp4_route) marks the shared
 * array as failed for the rest of the process: every later call then returns ids -1,
 * weights 0 and y = 0.
 * Errors: as moe_fp4_moe_forward, and TOO_LARGE; HIP if the array's address cannot be
 * obtained on the current device. */
#define MOE_FP4_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int moe_fp4_moe_forward_noalloc(const uint16_t* x, const uint16_t* w_router, int T, int hidden,
                                int n_experts, int k, const void* packed, int inter,
                                int32_t* topk_ids, float* topk_w, uint16_t* y, void* stream);

/* ------------------------------------------------------------------------------------
 * Layer chaining, for stacks of MoE layers (a harness step of the multi-layer decode
 * workload: RMSNorm is among the per-layer kernels of a decode step, [A100-FP4], section
 * 然后又发现每 token 启动 2000 次内核; residual and unit gain are the plain reading).
 * moe_fp4_residual_init:    residual [T x hidden] fp32 = x [T x hidden] bf16.
 * moe_fp4_residual_rmsnorm: residual += y (bf16, fp32 add), then
 *                           x_out = bf16_rne(residual / sqrt(mean(residual^2) + eps)),
 *                           the mean of squares accumulated in fp64; residual is updated
 *                           in place, x_out may not alias y.
 * moe_fp4_residual_rmsnorm needs hidden % 8 == 0 and hidden <= 16384 (BAD_SHAPE) and
 * 16-byte aligned arrays; moe_fp4_residual_init needs residual 4-byte and x 2-byte
 * alignment. Errors: INVALID_ARG, BAD_SHAPE, MISALIGNED, HIP.
 * ------------------------------------------------------------------------------------ */
int moe_fp4_residual_init(const uint16_t* x, float* residual, int T, int hidden, void* stream);

/* The next layer's routing straight from the residual stream, for chained layers:
 * residual_out = residual_in + y_prev (fp32 add), x_out = bf16_rne(residual_out /
 * sqrt(mean(residual_out^2) + eps)) (the same bits as moe_fp4_residual_rmsnorm), then the
 * top-k routing of x_out exactly as moe_fp4_route. At T == 1 this is one launch: every
 * workgroup of the router kernel normalises the row itself, so the separate norm launch of
 * a decode step goes away ([A100-FP4], section 然后又发现每 token 启动 2000 次内核: per-token
 * launches cost more than their math). residual_in, residual_out [T x hidden] fp32;
 * y_prev, x_out [T x hidden] bf16; no output (residual_out, x_out) may overlap an input
 * (residual_in, y_prev) or the other output: at T == 1 every workgroup reads the whole
 * input rows while the others write their slices of the outputs, so x_out cannot reuse
 * y_prev's buffer (INVALID_ARG). eps >= 0 and finite; the workspace as for
 * moe_fp4_route (its first 16 KB carry the synchronisation words between calls). hidden % 32
 * == 0 and <= 16384; 16-byte alignment except topk_ids / topk_w (4).
 * Errors: INVALID_ARG (null, eps, overlap, T / k / n_experts as moe_fp4_route), BAD_SHAPE,
 * MISALIGNED, WORKSPACE, HIP. */
int moe_fp4_route_residual(const float* residual_in, const uint16_t* y_prev, float* residual_out,
                           uint16_t* x_out, float eps, const uint16_t* w_router, int T, int hidden,
                           int n_experts, int k, int32_t* topk_ids, float* topk_w, void* workspace,
                           size_t workspace_bytes, void* stream);
int moe_fp4_residual_rmsnorm(float* residual, const uint16_t* y, uint16_t* x_out, int T,
                             int hidden, float eps, void* stream);

/* ------------------------------------------------------------------------------------
 * Dense FP8 weights: the shared expert and the dense projections. [A100-FP4], Chinese
 * translation, section A100 也没有 FP8: the dense weights are FP8 E4M3, kept as a storage
 * format; they go from memory into registers and become bf16 matrix-core operands there,
 * never expanded in memory. Format taken here: E4M3 "FN" codes (bit 7 sign, 4 exponent bits
 * with bias 7, 3 mantissa bits, 0x7F / 0xFF NaN, no infinities) of a row-major [rows x cols]
 * matrix (out x in) with one fp32 multiplier per 128 x 128 block (row-major
 * [ceil(rows / 128) x ceil(cols / 128)]): W[n][k] = e4m3(code) * multiplier. rows and cols
 * are multiples of 32, at most 16384. Products are exact (E4M3 fits bf16), sums are fp32
 * (one per 128-element chunk, scaled by its multiplier), outputs are rounded to bf16.
 * ------------------------------------------------------------------------------------ */

/* Bytes of one packed FP8 matrix (0 for an invalid shape). */
size_t moe_fp4_fp8_packed_bytes(int rows, int cols);

/* Load-time re-layout of one FP8 matrix into the tile-major order the kernels read (codes
 * device, 16-byte aligned; scale_inv device fp32; packed device, 16-byte aligned, of
 * moe_fp4_fp8_packed_bytes bytes). Errors: INVALID_ARG (null), BAD_SHAPE, MISALIGNED,
 * WORKSPACE (packed_bytes too small), HIP. */
int moe_fp4_fp8_pack(const uint8_t* codes, const float* scale_inv, int rows, int cols, void* packed,
                     size_t packed_bytes, void* stream);

/* Dense projection y [T x rows] = x [T x cols] W^T (bf16 in and out, device buffers,
 * 16-byte aligned; packed from moe_fp4_fp8_pack). Up to four tokens share one read of the
 * weights. T = 0 is a no-op. Errors: INVALID_ARG, BAD_SHAPE, MISALIGNED, HIP. */
int moe_fp4_fp8_linear(const uint16_t* x, int T, const void* packed, int rows, int cols,
                       uint16_t* y, void* stream);

/* h [T x inter] = bf16(silu(x W_gate^T) * (x W_up^T)) for x [T x hidden] and packed FP8 gate
 * and up [inter x hidden]. Errors: as moe_fp4_fp8_linear. */
int moe_fp4_fp8_swiglu(const uint16_t* x, int T, const void* gate, const void* up, int inter,
                       int hidden, uint16_t* h, void* stream);

/* The shared expert: y [T x hidden] = W_down h with h from moe_fp4_fp8_swiglu (two launches;
 * h goes to the workspace, moe_fp4_shared_expert_workspace_bytes(T, inter) bytes, 16-byte
 * aligned). The caller adds y to the routed experts' output. Errors: as moe_fp4_fp8_linear,
 * and WORKSPACE. */
size_t moe_fp4_shared_expert_workspace_bytes(int T, int inter);
int moe_fp4_shared_expert(const uint16_t* x, int T, const void* gate, const void* up,
                          const void* down, int hidden, int inter, uint16_t* y, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Speculative expert prefetch, opt-in ([8GB-GPU], section 提速之路：v1 到 v4, v4: the router
 * of layer l + 1 applied to layer l's input predicts the next layer's experts, which are
 * fetched ahead of need). The experts are resident in HBM here, so this reads the chosen
 * matrices of the experts ids[0 .. n_ids - 1] (device int32; ids outside [0, n_experts)
 * skipped) of a packed buffer with cached loads, which leaves them in the memory-side cache
 * every HBM read passes through (256 MB on MI355X), for a later FFN call to read from there.
 * matrices: bit 0 gate, bit 1 up, bit 2 down (codes and scales of each). Nothing is written
 * except, practically never, the device uint32 *sink (it keeps the loads alive; its
 * contents carry no meaning). Meant to run on a second stream while the HBM is idle (the
 * batch-1 route); the FFN's results do not depend on it. n_ids = 0 is a no-op.
 * Errors: INVALID_ARG (null, n_ids < 0 or > 65536, matrices not in 1..7), BAD_SHAPE,
 * MISALIGNED (ids and sink 4-byte, packed 16-byte), HIP. */
int moe_fp4_prefetch_experts(const int32_t* ids, int n_ids, const void* packed, int n_experts,
                             int hidden, int inter, int matrices, uint32_t* sink, void* stream);

/* Debug helper: counts the entries of topk_ids [T x k] outside [0, n_experts) into
 * *bad_count (a device int32 that this call overwrites). */
int moe_fp4_validate_ids(const int32_t* topk_ids, int T, int k, int n_experts,
                         int32_t* bad_count, void* stream);

/* Debug helper: dequantises matrix `matrix` (0 gate, 1 up, 2 down) of expert `expert` of
 * a packed buffer to fp32 out [rows x K] (gate/up: [inter x hidden], down: [hidden x
 * inter]) with the in-register decode the decode and small-M FFN kernels feed to their
 * matrix cores (the same device function): the FP4 -> bf16 conversion with the ue8m0 byte
 * as its scale, each bf16 widened exactly to fp32. out = E2M1(code) * 2^(e-127) rounded to
 * bf16, which is exact for every e = 0..254 (bf16 subnormals included) except where the
 * magnitude reaches 2^128 (e = 253 with |E2M1| >= 4, e = 254 with |E2M1| >= 2: +-inf);
 * NaN for e = 255 ([8GB-GPU], section RTX 50xx 上的三个从不抛错的 Bug: ue8m0 scales; 255 as
 * NaN is the E8M0 reading). The grouped path hands the same bytes to the block-scaled
 * matrix cores, which apply them as E8M0 scales themselves.
 * Errors: INVALID_ARG (null, expert or matrix out of range), BAD_SHAPE, MISALIGNED, HIP. */
int moe_fp4_debug_dequant(const void* packed, int n_experts, int hidden, int inter, int expert,
                          int matrix, float* out, void* stream);

/* Debug helper: the grouped path's activation quantisation of x [T x hidden] bf16 (device),
 * decoded back to fp32 out [T x hidden] (device): per 32-element block, terms 1: one MXFP8
 * E4M3 term (the GROUPED_FP8 path's operand); terms 2: two MXFP6 E2M3 terms (the GROUPED
 * path's: hi, then lo = the same quantisation of x - hi), with one ue8m0 scale each, the
 * scale the smallest power of two that fits the block's maximum in the format's largest
 * value (448 for E4M3, 7.5 for E2M3), codes rounded to nearest with ties to the even code
 * ([8GB-GPU], section RTX 50xx 上的三个从不抛错的 Bug: ue8m0-scaled activations). This scale
 * rule is the library's own reading, not the OCP MX one (2^(floor(log2 max) - emax) with
 * clipping): where the block maximum's significand exceeds the largest value's (1.75 for
 * E4M3, 1.875 for E2M3) it takes the next power of two, so no element is clipped. out is the exact sum of the decoded terms. workspace:
 * moe_fp4_debug_act_quant_bytes(T, hidden) bytes of device memory, 16-byte aligned, contents
 * irrelevant. Errors: INVALID_ARG (null pointer, T < 0, terms not 1 or 2), BAD_SHAPE,
 * MISALIGNED, WORKSPACE, HIP. */
size_t moe_fp4_debug_act_quant_bytes(int T, int hidden);
int moe_fp4_debug_act_quant(const uint16_t* x, int T, int hidden, int terms, void* workspace,
                            size_t workspace_bytes, float* out, void* stream);

/* Measurement helper (not on the FFN path): reads `bytes` bytes at src with 16-byte
 * non-temporal loads, the load form of the expert kernels, over a grid of up to 2048
 * workgroups; for the measured HBM streaming peak. src: device, 16-byte aligned; bytes a
 * positive multiple of 16. sink: one device uint32 that the kernel writes only when the
 * XOR of everything read equals a fixed constant (it keeps the loads; the contents of sink
 * carry no meaning). Errors: INVALID_ARG (null pointer, bytes 0 or not a multiple of 16),
 * MISALIGNED, HIP. */
int moe_fp4_debug_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Measurement helper (not on the FFN path): n_workgroups workgroups of four wavefronts,
 * each wavefront issuing iters x MOE_FP4_PROBE_MFMA_CHAINS independent block-scaled
 * 16x16x128 matrix-core operations (v_mfma_scale_f32_16x16x128_f8f6f4; 2 x 16 x 16 x 128
 * flops each) with B in FP4 E2M1 and A in FP4 E2M1 (fmt_a = 4) or FP8 E4M3 (fmt_a = 0),
 * operands held in registers; for the measured matrix-core peak. sink as above.
 * Errors: INVALID_ARG (null sink, fmt_a not 0 or 4, n_workgroups or iters outside
 * [1, 1 << 20]), HIP. */
#define MOE_FP4_PROBE_MFMA_CHAINS 8
int moe_fp4_debug_mfma_loop(int fmt_a, int n_workgroups, int iters, uint32_t* sink,
                            void* stream);

/* ------------------------------------------------------------------------------------
 * Built-in kernel timing, for measurement. When enabled, every kernel the library
 * launches is bracketed by a pair of HIP events on the launch stream (host-side event
 * objects created here; no device memory). moe_fp4_timing_read synchronises on the
 * recorded events and returns, for one kernel kind, the number of launches and the
 * summed GPU time in milliseconds since the last reset. Kinds are the MOE_FP4_KERNEL_*
 * values. Not thread-safe; meant for single-threaded benchmarks.
 * ------------------------------------------------------------------------------------ */
#define MOE_FP4_KERNEL_PACK 0
#define MOE_FP4_KERNEL_ROUTER_GEMV 1
#define MOE_FP4_KERNEL_TOPK 2
#define MOE_FP4_KERNEL_GATE_UP 3
#define MOE_FP4_KERNEL_DOWN_COMBINE 4
#define MOE_FP4_KERNEL_ROUTE_DECODE 5 /* batch-1 router GEMV + selection in one launch */
#define MOE_FP4_KERNEL_GROUPED_SORT 6
#define MOE_FP4_KERNEL_GROUPED_QUANT 7
#define MOE_FP4_KERNEL_GROUPED_GATE_UP 8
#define MOE_FP4_KERNEL_GROUPED_DOWN 9
#define MOE_FP4_KERNEL_GROUPED_COMBINE 10
#define MOE_FP4_KERNEL_NORM 11 /* residual init and residual + RMSNorm */
#define MOE_FP4_KERNEL_PROBE_STREAM 12 /* moe_fp4_debug_stream_read */
#define MOE_FP4_KERNEL_PROBE_MFMA 13   /* moe_fp4_debug_mfma_loop */
#define MOE_FP4_KERNEL_SMALL_M_GATE_UP 14
#define MOE_FP4_KERNEL_SMALL_M_DOWN 15
#define MOE_FP4_KERNEL_FP8_GEMV 16     /* moe_fp4_fp8_linear, _swiglu, _shared_expert */
#define MOE_FP4_KERNEL_PREFETCH 17     /* moe_fp4_prefetch_experts */
#define MOE_FP4_KERNEL_KINDS 18

int moe_fp4_timing_enable(int enable);
int moe_fp4_timing_reset(void);
int moe_fp4_timing_read(int kind, int* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP4_H */
