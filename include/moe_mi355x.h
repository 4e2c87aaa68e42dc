/*
 * moe_mi355x.h -- C ABI of the fused sparse Mixture-of-Experts layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer, as the pages define it:
 *   [MoE]     mini-sglang guide, chapter 7 (models, MoE backend, kernel
 *             infrastructure), paragraph on the MoE routing layer: a router
 *             linear gives per-expert logits, the top-k experts are chosen
 *             as torch.topk does, and the k expert outputs are weighted by
 *             their softmax scores and summed; paragraph on the fused
 *             backend: tokens are grouped by their assigned expert so each
 *             expert's weights are read with coalesced accesses.
 *   [Linear]  handbook page "The op layer: BaseOP and the layers", section
 *             "Linear layers": a linear layer is y = x W^T (+ b); the MoE
 *             router is replicated, not sharded.
 *   [Models]  handbook page "Models and weight loading": section
 *             "ModelConfig" (num_experts, num_experts_per_tok,
 *             moe_intermediate_size, norm_topk_prob), section "Model
 *             structure" (each expert is a GatedMLP: merged gate_up
 *             projection, silu(gate) * up, down projection; only silu) and
 *             section "Streaming weight loading" (per-expert weights stacked
 *             into [E, ...]; gate and up merged in that order).
 *
 * The layer is five calls, in this order, on one stream:
 *   moe_route -> moe_align_by_expert -> moe_grouped_gemm_gate_up_silu ->
 *   moe_grouped_gemm_down -> moe_combine
 * No residual is added (the decoder adds it outside the MLP). The expert
 * weights are converted once, when they are loaded, by moe_pack_weights into
 * the layout the grouped GEMMs stream.
 *
 * Conventions for every call
 *  - Pointers named as device pointers must point to device memory of the
 *    current HIP device; the caller allocates and owns every buffer. The
 *    library allocates nothing, frees nothing and keeps no pointer after the
 *    call returns.
 *  - All tensors are dense and row-major. bf16 tensors are passed as void*
 *    holding raw bfloat16 bit patterns; fp32 as float*; indices as int32_t*.
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *    enqueues work: it never synchronises and never reads device memory on
 *    the host. Arguments are validated on the host before anything is
 *    enqueued; a call that fails validation enqueues nothing.
 *  - Return value: MOE_OK, or a negative MOE_ERR_* code. moe_last_error()
 *    returns a thread-local message describing the last failure.
 *  - Limits: 1 <= E <= 256, 1 <= k <= min(E, 32), H % 64 == 0, I % 32 == 0,
 *    T >= 0 (T == 0 is a successful no-op), T * k < 2^31,
 *    block_m in {16, 32, 64, 128, 256} (256: the grouping pads each expert to
 *    256 rows and the GEMMs compute each such block as two 128-row tiles, so
 *    every output equals block_m 128's bit for bit); with block_m 64 or more
 *    the grouped GEMMs' activation operand (x: T*H*2 bytes; act: cap*I*2
 *    bytes) and one expert's weights must each be under 4 GiB (the copies use
 *    32-bit offsets).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3

#define MOE_OK 0
#define MOE_ERR_INVALID (-1)     /* null required pointer, negative size, bad enum */
#define MOE_ERR_UNSUPPORTED (-2) /* shape outside the limits above */
#define MOE_ERR_HIP (-3)         /* HIP launch/configuration error */
#define MOE_ERR_WORKSPACE (-4)   /* workspace or capacity too small */

/* Element types of the tensors whose type a call takes as an argument. */
#define MOE_DTYPE_BF16 0
#define MOE_DTYPE_FP32 1
#define MOE_DTYPE_FP16 2
#define MOE_OUT_BF16 MOE_DTYPE_BF16
#define MOE_OUT_FP32 MOE_DTYPE_FP32

/* Size of the static device scratch of moe_align_by_expert_noalloc. */
#define MOE_ALIGN_NOALLOC_MAX_WORKSPACE_BYTES 262144

/* Version of this ABI (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Message for the last failing call on this thread ("" if none). The string
 * is owned by the library and valid until the next call on this thread. */
const char* moe_last_error(void);

/*
 * Router linear, softmax, top-k and optional renormalisation ([MoE],
 * [Linear], [Models] norm_topk_prob).
 *
 *   x            [T, H] bf16, device. May be NULL: then `logits` is an input.
 *   w_router     [E, H] bf16, device (ignored when x is NULL).
 *   router_bias  [E] fp32, device, or NULL for no bias (ignored when x is NULL).
 *   logits       [T, E] fp32, device. Output when x != NULL:
 *                logits[t,e] = sum_h x[t,h] * w_router[e,h] + bias[e],
 *                accumulated in fp32. Input when x == NULL.
 *   topk_ids     [T, k] int32, device, output: the k experts with the largest
 *                logits (equivalently the largest softmax scores), in
 *                descending order; equal logits -> lower expert index first.
 *   topk_weights [T, k] fp32, device, output: softmax over all E experts at
 *                the selected experts; if norm_topk_prob != 0, divided by
 *                their sum over the k selected experts (then they sum to 1).
 * Selection is decided on the fp32 logits, so given the same logits it is
 * exact and reproducible.
 */
int moe_route(const void* x, const void* w_router, const float* router_bias, float* logits, int32_t* topk_ids,
              float* topk_weights, int64_t T, int32_t H, int32_t E, int32_t k, int32_t norm_topk_prob,
              void* stream);

/*
 * Rows of the expert-grouped permutation sufficient for any routing of T
 * tokens: T*k real rows plus at most block_m-1 pad rows for each non-empty
 * expert, rounded up to block_m. Returns -1 on invalid arguments.
 */
int64_t moe_align_capacity(int64_t T, int32_t k, int32_t E, int32_t block_m);

/* Bytes of device workspace moe_align_by_expert needs (per-tile expert
 * histograms). Returns 0 when none is needed or the arguments are invalid. */
size_t moe_align_workspace_bytes(int64_t T, int32_t k, int32_t E, int32_t block_m);

/*
 * Group (token, slot) pairs by assigned expert ([MoE], fused-backend
 * paragraph), padded to the GEMM row tile.
 *
 *   topk_ids      [T, k] int32, device, input (values in [0, E)).
 *   cap           = moe_align_capacity(T, k, E, block_m) rows (not passed:
 *                   the output buffers must have at least these sizes).
 *   sorted_ids    [cap] int32, device, output. The flat index i = t*k + j of
 *                 slot j of token t. Expert e owns rows
 *                 [off_e, off_e + pad_e), pad_e = ceil(c_e/block_m)*block_m,
 *                 c_e = number of pairs routed to e, off_e = sum of pad_e'
 *                 for e' < e. Its first c_e rows hold its flat indices in
 *                 ascending order; its other rows, and every row from
 *                 num_padded on, hold the sentinel T*k.
 *   block_expert  [cap / block_m] int32, device, output: owner expert of
 *                 each block_m-row block, -1 for blocks from num_padded on.
 *                 Experts with no pairs own no block.
 *   expert_counts [E] int32, device, output: c_e.
 *   num_padded    [1] int32, device, output: sum of pad_e.
 *   workspace     device scratch of at least moe_align_workspace_bytes(...)
 *                 bytes (may be NULL when that is 0); contents on entry are
 *                 ignored.
 * The result is deterministic (no order-dependent atomics).
 */
int moe_align_by_expert(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t block_m,
                        int32_t* sorted_ids, int32_t* block_expert, int32_t* expert_counts, int32_t* num_padded,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_align_by_expert without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, results and guarantees as
 * moe_align_by_expert; the per-tile histograms go to a static device array of
 * MOE_ALIGN_NOALLOC_MAX_WORKSPACE_BYTES (256 KB) that each GPU the
 * library runs on holds until the process ends. The call allocates and frees
 * nothing. Calls whose moe_align_workspace_bytes(T, k, E, block_m) exceeds
 * MOE_ALIGN_NOALLOC_MAX_WORKSPACE_BYTES (more than 65536 / E tiles: T*k above about 1M pairs at E = 256)
 * return MOE_ERR_UNSUPPORTED and enqueue nothing. Every call on one GPU uses
 * the same array: calls that may overlap on one GPU (different streams, or
 * host threads enqueueing concurrently) race and must be serialised by the
 * caller. The first call on each device looks up that device's copy of the
 * array (hipGetSymbolAddress) and may return MOE_ERR_HIP if that fails.
 */
int moe_align_by_expert_noalloc(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t block_m,
                                int32_t* sorted_ids, int32_t* block_expert, int32_t* expert_counts,
                                int32_t* num_padded, void* stream);

/* Bytes of a packed [E, N, K] bf16 weight (equal to the row-major size), or
 * 0 when the shape cannot be packed (needs N % 16 == 0 and K % 32 == 0). */
size_t moe_packed_weight_bytes(int32_t E, int32_t N, int32_t K);

/*
 * Convert expert weights from the row-major layout they are loaded in
 * ([Models], "Streaming weight loading": per-expert tensors stacked into
 * [E, N, K]) into the fragment layout the grouped GEMMs read. Done once per
 * weight, outside the layer.
 *
 *   w         [E, N, K] bf16, device, row-major. For the merged gate/up
 *             weight (gated != 0) N = 2I with rows 0..I-1 gate and I..2I-1
 *             up; for the down weight (gated == 0) N = H, K = I.
 *   w_packed  device buffer of moe_packed_weight_bytes(E, N, K) bytes,
 *             output; must not overlap w.
 * Layout of w_packed: each expert's rows are cut into 16-row bands and each
 * band into 32-column k-steps; block (band, k-step) is 512 contiguous bf16 in
 * which elements 8l..8l+7 hold row l%16 of the band at columns 8*(l/16) ..
 * 8*(l/16)+7 of the k-step (l = 0..63). Blocks are ordered expert, band,
 * k-step. When gated, packed band 2b is gate band b (rows 16b..16b+15) and
 * packed band 2b+1 is up band b (rows I+16b..I+16b+15).
 */
int moe_pack_weights(const void* w, void* w_packed, int32_t E, int32_t N, int32_t K, int32_t gated, void* stream);

/*
 * Grouped gate/up projection with fused SiLU-and-mul ([Models], "Model
 * structure": gate_up_proj, then silu(gate) * up). For every row r below
 * num_padded whose sorted_ids[r] = i is not the sentinel, with token
 * t = i / k and expert e = block_expert[r / block_m]:
 *   g_c = sum_h x[t,h] * w13[e, c, h],  u_c = sum_h x[t,h] * w13[e, I + c, h]
 *   act[r, c] = bf16(silu(g_c) * u_c),  silu(z) = z / (1 + exp(-z)),
 * with bf16 products accumulated in fp32 on the matrix cores. Pad rows are
 * written as zeros. Rows from num_padded on are not touched.
 *
 *   x          [T, H] bf16, device.
 *   w13        [E, 2I, H] bf16, device, packed by moe_pack_weights (gated = 1)
 *              from the row-major weight whose rows 0..I-1 are gate and
 *              I..2I-1 up; w13[e, c, h] above refers to that row-major
 *              weight.
 *   sorted_ids, block_expert, num_padded: from moe_align_by_expert with the
 *              same T, k, E, block_m; cap = moe_align_capacity(...).
 *   act        [cap, I] bf16, device, output: rows in sorted order, stored
 *              as MFMA fragment blocks like the packed weights (16-row x
 *              32-column blocks of 512 elements, row-band major; element
 *              (r, c) at ((r/16)*(I/32) + c/32)*512 + (16*((c%32)/8) + r%16)*8
 *              + c%8), so the down projection reads 1 KB blocks. Rows below
 *              num_padded occupy the first num_padded*I elements.
 */
int moe_grouped_gemm_gate_up_silu(const void* x, const void* w13, const int32_t* sorted_ids,
                                  const int32_t* block_expert, const int32_t* num_padded, int64_t T, int32_t k,
                                  int32_t H, int32_t I, int32_t E, int32_t block_m, int64_t cap, void* act,
                                  void* stream);

/*
 * Grouped down projection ([Models], "Model structure": down_proj). For
 * every row r below num_padded with sorted_ids[r] = i not the sentinel and
 * e = block_expert[r / block_m]:
 *   y[i, h] = sum_c act[r, c] * w2[e, h, c]
 * accumulated in fp32 and stored as y_dtype: MOE_DTYPE_FP16 (IEEE half,
 * round to nearest even: 11 significant bits, so the layer's error stays
 * dominated by the final bf16 rounding of the output, at half the bytes of
 * fp32; values beyond +-65504 become +-inf) or MOE_DTYPE_FP32. Every one of
 * the T*k rows of y is written exactly once; pad rows of act are never used
 * for a real row.
 *
 *   act      [cap, I] bf16, device, in the fragment-block layout written by
 *            moe_grouped_gemm_gate_up_silu.
 *   w2       [E, H, I] bf16, device, packed by moe_pack_weights (gated = 0);
 *            w2[e, h, c] above refers to the row-major weight.
 *   y        [T*k, H] fp16 or fp32, device, output, in (token, slot) order.
 *   y_dtype  MOE_DTYPE_FP16 or MOE_DTYPE_FP32 (anything else: MOE_ERR_INVALID).
 */
int moe_grouped_gemm_down(const void* act, const void* w2, const int32_t* sorted_ids, const int32_t* block_expert,
                          const int32_t* num_padded, int64_t T, int32_t k, int32_t H, int32_t I, int32_t E,
                          int32_t block_m, int64_t cap, void* y, int32_t y_dtype, void* stream);

/*
 * moe_grouped_gemm_down and moe_combine in one launch ([MoE]: the expert
 * outputs weighted by their scores and summed, at the end of the layer):
 * the down projection stores each expert output row in y as
 * moe_grouped_gemm_down does, and the weighted sum of a token's k rows is
 * formed, inside the same kernel, by the workgroup that completes the
 * token's last slot for a group of 128 output columns (a device-scope
 * arrival count per (token, group) with release/acquire ordering). out is
 * computed exactly as moe_combine computes it (fp32, slots in order), so it
 * does not depend on which workgroup sums a group: every output is
 * bit-for-bit reproducible.
 *
 *   topk_weights  [T, k] fp32, device (as for moe_combine).
 *   y             [T*k, H], device, y_dtype (fp16 or fp32), written as by
 *                 moe_grouped_gemm_down and read back by the kernel.
 *   counters      [moe_combine_counter_count(T, H)] int32, device: must be all
 *                 zero on entry; every call that returns MOE_OK leaves them
 *                 zero (zero them once when allocating).
 *   out           [T, H], device: bf16 (out_dtype MOE_OUT_BF16, round to
 *                 nearest even) or fp32 (MOE_OUT_FP32).
 *   (the rest)    as moe_grouped_gemm_down.
 * Two calls sharing counters must not overlap in time.
 */
int moe_grouped_gemm_down_combine(const void* act, const void* w2, const int32_t* sorted_ids,
                                  const int32_t* block_expert, const int32_t* num_padded, const float* topk_weights,
                                  int64_t T, int32_t k, int32_t H, int32_t I, int32_t E, int32_t block_m, int64_t cap,
                                  void* y, int32_t y_dtype, int32_t* counters, void* out, int32_t out_dtype,
                                  void* stream);

/* Number of int32 counters moe_grouped_gemm_down_combine needs: T times the
 * number of 128-column groups of H. -1 on invalid arguments. */
int64_t moe_combine_counter_count(int64_t T, int32_t H);

/*
 * Weighted sum of the k expert outputs of each token ([MoE]: expert outputs
 * weighted by their scores and summed):
 *   out[t, h] = sum_j topk_weights[t, j] * y[t*k + j, h]   (fp32 accumulation,
 *                                                          j = 0, 1, ... in order)
 *
 *   y             [T*k, H], device, MOE_DTYPE_FP16 or MOE_DTYPE_FP32 as y_dtype.
 *   topk_weights  [T, k] fp32, device.
 *   out           [T, H], device: bf16 (round to nearest even) when
 *                 out_dtype == MOE_OUT_BF16, fp32 when MOE_OUT_FP32.
 */
int moe_combine(const void* y, int32_t y_dtype, const float* topk_weights, int64_t T, int32_t k, int32_t H,
                void* out, int32_t out_dtype, void* stream);

/*
 * Fused residual add + RMSNorm, the step that precedes the MoE layer in a
 * decoder layer (handbook page "The op layer: BaseOP and the layers",
 * section "Ops: reference implementations and dispatch" for rmsnorm and
 * fused_add_rmsnorm, section "RMSNorm and the residual" for the fused op and
 * the first-layer case). In place, on [T, H] bf16 rows:
 *   has_residual != 0:  residual <- bf16(residual + x)   (fp32 add)
 *   has_residual == 0:  residual <- x                   (first layer)
 *   x <- bf16(weight * bf16(residual / sqrt(mean(residual^2) + eps)))
 * (the norm in fp32; the normalized value is cast to bf16 before the
 * weight multiply, as the reference op does). The normalized x is the
 * layer's input; residual carries the new residual stream.
 *
 *   x         [T, H] bf16, device, in/out.
 *   residual  [T, H] bf16, device, in/out (input ignored when has_residual
 *             is 0); must not alias x.
 *   weight    [H] bf16, device.
 * Limits: H a multiple of 8, at most 16384; eps >= 0. T == 0 is a no-op.
 */
int moe_fused_add_rmsnorm(void* x, void* residual, const void* weight, int64_t T, int32_t H, float eps,
                          int32_t has_residual, void* stream);

/*
 * The residual add + RMSNorm that precedes the layer fused into the router's
 * read of x (handbook page "The op layer: BaseOP and the layers", sections
 * "Ops: reference implementations and dispatch" and "RMSNorm and the
 * residual"), then moe_route on the normalized rows. Equivalent to
 * moe_fused_add_rmsnorm on copies of x and residual followed by moe_route:
 *   residual_out = bf16(residual + x)   (fp32 add; = x when has_residual == 0)
 *   x_out = bf16(norm_weight * bf16(residual_out / sqrt(mean(residual_out^2) + eps)))
 *   logits, topk_ids, topk_weights as moe_route(x_out, w_router, ...)
 * The router reads x and the residual once per row and writes x_out and
 * residual_out once, instead of a separate normalization pass over [T, H].
 * The mean and square root are taken in fp32 with the same summation order
 * for every batch size, so a row's outputs do not depend on T.
 *
 *   x             [T, H] bf16, device, input.
 *   residual      [T, H] bf16, device, input (ignored, may be NULL, when
 *                 has_residual == 0: the first layer).
 *   norm_weight   [H] bf16, device.
 *   x_out         [T, H] bf16, device, output: the layer's input.
 *   residual_out  [T, H] bf16, device, output: the new residual stream.
 *   (the rest)    as moe_route; x_out is what the grouped gate/up GEMM then
 *                 reads.
 * Every router workgroup of a block of tokens reads that block's rows, so the
 * outputs cannot be written in place: x_out and residual_out must not overlap
 * each other, x or residual (MOE_ERR_INVALID). Limits: those of moe_route and
 * H <= 16384; eps >= 0.
 */
int moe_fused_add_rmsnorm_route(const void* x, const void* residual, const void* norm_weight, float eps,
                                int32_t has_residual, void* x_out, void* residual_out, const void* w_router,
                                const float* router_bias, float* logits, int32_t* topk_ids, float* topk_weights,
                                int64_t T, int32_t H, int32_t E, int32_t k, int32_t norm_topk_prob, void* stream);

/* The block_m the library's GEMMs run fastest with for this routing shape.
 * A tile-size choice only: for a fixed block_m every result is bit-for-bit
 * reproducible and independent of the other tokens in the batch; different
 * block_m values use different matrix-core instruction shapes (16x16x32 for
 * 16 and 32, 32x32x16 for 64 and 128), whose fp32 accumulation orders differ,
 * so their outputs agree to rounding, not bit for bit. Returns -1 on invalid
 * arguments. */
int32_t moe_pick_block_m(int64_t T, int32_t k, int32_t E);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
