/*
 * libmoe -- routed-expert MoE layer (Kimi-K2 shapes) on AMD Instinct MI355X (gfx950).
 *
 * The layer: given normalised features x[N][d] (bfloat16) and, per token, K
 * expert ids and routing weights over E experts, run each token through its K
 * selected SwiGLU experts, y = down(silu(gate x) * up x), and return the
 * routing-weighted sum of their outputs (plus, optionally, one shared expert
 * applied to every token).
 *   - The layer, dispatch and combine: Open Model Atlas, "Kimi K2 - Mixture of
 *     experts" page (experts inspector): Code (moe_infer, forward) and Direct
 *     evidence "moe-forward" (router-weighted sum plus the shared expert;
 *     tokens sorted by expert, each expert run on its slice, outputs scattered
 *     back).
 *   - The expert: "SwiGLU output" page, evidence "mlp" (DeepseekV3MLP: three
 *     bias-free linear maps, weight[out][in]); "Element-wise product" page,
 *     formula h = a (.) u with a = silu(gate x), u = up x.
 *   - FP8 storage: "Input features" page, evidence "linear"
 *     (quantization_config: e4m3, weight_block_size [128, 128], dynamic
 *     activation scheme).
 *
 * The layer is split into three calls, in this order on one stream:
 *   moe_dispatch -> moe_grouped_swiglu -> moe_combine.
 * The shared expert is moe_grouped_swiglu with E = 1, K = 1 and the identity
 * dispatch (moe_dispatch of an all-zero ids[N][1] with E = 1); its output is
 * passed as `shared` to moe_combine.
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers owned by the caller. The library
 *     never allocates device memory; scratch lives in a caller-provided
 *     workspace whose size the *_workspace_size queries return.
 *   - All work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *     the default stream). No host synchronisation happens unless a flag asks
 *     for it (MOE_FLAG_CHECKED).
 *   - Arrays are row-major and dense. bfloat16 and e4m3 arrays must be
 *     16-byte aligned (they are moved with 16-byte vector accesses); int32 and
 *     float32 arrays 4-byte aligned.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     non-MOE_OK status means nothing was enqueued (except MOE_ERR_BAD_ID,
 *     MOE_ERR_DUP_ID and MOE_ERR_HIP, reported after the work ran).
 *   - Outputs must not alias inputs. Calls that share a workspace must be
 *     ordered (same stream or synchronised).
 *   - Numbers: e4m3 is the OCP FP8 E4M3FN format (bias 7, max 448, no inf);
 *     bfloat16 is stored as its 16-bit pattern. Dequantised value = code *
 *     scale. Scales are float32. Wherever values are quantised to e4m3 (x, and
 *     the product h inside the grouped SwiGLU calls): a group's scale comes
 *     from its largest non-NaN magnitude, a scaled value beyond +-448
 *     saturates to +-448, and a NaN value (including inf / inf in a group
 *     whose largest magnitude is infinite) gets a NaN code (0x7F or 0xFF; the
 *     sign of a NaN code is unspecified).
 *   - No entry point uses floating-point atomics; results are bit-identical
 *     from run to run for the same inputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL */
    MOE_ERR_SHAPE = 2,       /* a size is out of range (see each call) */
    MOE_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
    MOE_ERR_WORKSPACE = 4,   /* workspace smaller than the size query returned */
    MOE_ERR_BAD_ID = 5,      /* checked mode: an expert id outside [0, E) */
    MOE_ERR_DUP_ID = 6,      /* checked mode: an id repeated within one token's row */
    MOE_ERR_HIP = 7,         /* a HIP runtime call failed; see moe_last_hip_error() */
    MOE_ERR_DEVICE = 8       /* the current device is not a gfx950 GPU */
} moe_status;

/* Validate expert ids on the device and wait for the result (one host sync). */
#define MOE_FLAG_CHECKED 1u
/* moe_grouped_swiglu: force the GEMM tile height (sorted rows of one expert per
 * workgroup) instead of choosing it from the expected rows per expert,
 * N*K / min(E, N*K). Results do not depend on it, bit for bit. Batches with
 * N*d or N*K*d_ff at or above 2^32 bytes always use 16-row tiles. */
#define MOE_FLAG_TILE_16 (1u << 4)
#define MOE_FLAG_TILE_128 (2u << 4)
#define MOE_FLAG_TILE_192 (3u << 4)
#define MOE_FLAG_TILE_256 (4u << 4)
#define MOE_FLAG_TILE_224 (5u << 4)
#define MOE_FLAG_TILE_MASK (7u << 4)

/* Limits (checked, MOE_ERR_SHAPE beyond them). */
#define MOE_MAX_EXPERTS 8192
#define MOE_MAX_TOPK 64
#define MOE_MAX_DIM 65536

/* ------------------------------------------------------------------------
 * Dispatch ("Mixture of experts" page, Code: moe_infer -- per-expert token
 * counts, the sort of flat slots by expert, the running start/end indices of
 * each expert's slice, and the inverse order used to scatter outputs back).
 *
 * A slot is one (token, choice) pair, s = n*K + k. Produces:
 *   counts[E]        tokens routed to each expert (tokens_per_expert);
 *   offsets[E+1]     offsets[0] = 0, offsets[e+1] = offsets[e] + counts[e];
 *                    expert e owns sorted positions [offsets[e], offsets[e+1]);
 *   sorted_slot[N*K] position -> slot, ascending expert, ties by ascending
 *                    slot (stable: the pages leave the tie order open);
 *   slot_pos[N*K]    slot -> position (inverse of sorted_slot).
 * topk_ids[N][K] int32. 0 <= N, N*K < 2^31; 1 <= K <= min(E, MOE_MAX_TOPK);
 * 1 <= E <= MOE_MAX_EXPERTS. N = 0 writes offsets (all zero) and counts only.
 * Ids must lie in [0, E) and be distinct within a row. Without
 * MOE_FLAG_CHECKED a violation gives unspecified (but memory-safe) outputs:
 * an out-of-range slot gets slot_pos = -1 and is left out. With it, the call
 * synchronises `stream` and returns MOE_ERR_BAD_ID or MOE_ERR_DUP_ID.
 * ---------------------------------------------------------------------- */
size_t moe_dispatch_workspace_size(int64_t N, int32_t K, int32_t E);

moe_status moe_dispatch(const int32_t* topk_ids, int64_t N, int32_t K, int32_t E,
                        int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                        int32_t* slot_pos, void* workspace, size_t workspace_bytes,
                        uint32_t flags, void* stream);

/* ------------------------------------------------------------------------
 * Grouped SwiGLU experts ("SwiGLU output" page, evidence "mlp";
 * "Element-wise product" page; FP8 format from "Input features" page,
 * evidence "linear").
 *
 * For every expert e and every sorted position p in [offsets[e], offsets[e+1])
 * with token n = sorted_slot[p] / K:
 *   xq = e4m3 quantisation of x[n], one scale per 128 features
 *        (scale = amax/448, code = e4m3(x/scale); an all-zero group has scale 1)
 *   g  = W_gate[e] xq,  u = W_up[e] xq         (d -> d_ff, per-128x128-block weight scales)
 *   h  = silu(g) * u, requantised to e4m3 per 128 features (same rule)
 *   y_sorted[p] = bfloat16(W_down[e] h)        (d_ff -> d), unweighted.
 * Accuracy delivered: each 128-wide block product of g and u (codes times codes)
 * is summed exactly up to float32 rounding; each block product of the down
 * projection is summed by the FP8 matrix op, which keeps about 14 bits below
 * its largest partial sum (an error of up to about 7e-5 of the block's sum of
 * |products|). Each block product is multiplied by its activation scale and
 * weight block scale and added to a float32 accumulator, blocks in K order;
 * silu uses the hardware exponential and reciprocal. A value of h close to an
 * e4m3 rounding midpoint can therefore take the neighbouring code. Against the
 * plain definition (exact dot products, exact silu), every token's output is
 * within a relative L2 error of 1e-2 on the tested shapes, d = 7168 with
 * d_ff = 2048 or 18432 and d_ff = 1024 with one choice per token among them
 * (the largest seen: 8.7e-3, one choice per token, d_ff = 2048).
 *
 * x[N][d] bf16. offsets[E+1], sorted_slot[N*K] as produced by moe_dispatch
 * for the same N, K, E (other contents give unspecified but memory-safe
 * results). Weights, stacked over experts, weight[out][in]:
 *   w_gate, w_up [E][d_ff][d] e4m3;  s_gate, s_up [E][d_ff/128][d/128] float32
 *   w_down [E][d][d_ff] e4m3;        s_down [E][d/128][d_ff/128] float32
 * y_sorted[N*K][d] bf16, in sorted-position order.
 * d and d_ff: positive multiples of 128, at most MOE_MAX_DIM; N, K and E as
 * moe_dispatch. N = 0 is a no-op. The workspace size queries return 0 for
 * arguments the call would reject.
 * ---------------------------------------------------------------------- */
size_t moe_swiglu_workspace_size(int64_t N, int32_t K, int32_t E, int32_t d, int32_t d_ff);

moe_status moe_grouped_swiglu(const uint16_t* x, int64_t N, int32_t K, int32_t E, int32_t d,
                              int32_t d_ff, const int32_t* offsets, const int32_t* sorted_slot,
                              const uint8_t* w_gate, const float* s_gate, const uint8_t* w_up,
                              const float* s_up, const uint8_t* w_down, const float* s_down,
                              uint16_t* y_sorted, void* workspace, size_t workspace_bytes,
                              uint32_t flags, void* stream);

/* ------------------------------------------------------------------------
 * moe_grouped_swiglu for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same call and the same result, bit for bit, with no
 * workspace argument. Its scratch (the quantised activations and product and
 * the tile list) lives in a fixed array inside the library, one per GPU,
 * MOE_NOALLOC_SCRATCH_BYTES long, held from the library's first use on a GPU
 * until the process ends. The call allocates nothing. A problem whose
 * moe_swiglu_workspace_size(N, K, E, d, d_ff) exceeds that size returns
 * MOE_ERR_WORKSPACE with nothing enqueued (at Kimi-K2 shapes, d = 7168,
 * d_ff = 2048, K = 8, E = 384: up to 2,760 tokens). Every call on a GPU uses that
 * GPU's one array: calls that may overlap in time on one GPU (different
 * streams without ordering between them) race on it and must not be made.
 * Nothing in the array needs clearing between calls: each call writes what it
 * reads. Other arguments, limits and errors as moe_grouped_swiglu.
 * ---------------------------------------------------------------------- */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

moe_status moe_grouped_swiglu_noalloc(const uint16_t* x, int64_t N, int32_t K, int32_t E,
                                      int32_t d, int32_t d_ff, const int32_t* offsets,
                                      const int32_t* sorted_slot, const uint8_t* w_gate,
                                      const float* s_gate, const uint8_t* w_up,
                                      const float* s_up, const uint8_t* w_down,
                                      const float* s_down, uint16_t* y_sorted, uint32_t flags,
                                      void* stream);

/* ------------------------------------------------------------------------
 * Grouped SwiGLU experts on activations already quantised: moe_grouped_swiglu
 * from its second step on, with xq/xs in place of the e4m3 quantisation of x.
 * For callers that produce the codes elsewhere: moe_rmsnorm_quantize_rows,
 * which quantises in the same pass as the block's RMSNorm, or one GPU of an
 * expert-parallel group that receives its tokens' rows already quantised.
 * xq[N][d] e4m3 codes and xs[N][d/128] float32 scales, laid out and defined
 * as moe_quantize_rows writes them; other arguments as moe_grouped_swiglu.
 * With xq, xs = moe_quantize_rows(x), y_sorted equals moe_grouped_swiglu's
 * bit for bit. The workspace needs moe_swiglu_q_workspace_size bytes (no room
 * for xq/xs).
 * ---------------------------------------------------------------------- */
size_t moe_swiglu_q_workspace_size(int64_t N, int32_t K, int32_t E, int32_t d, int32_t d_ff);

moe_status moe_grouped_swiglu_q(const uint8_t* xq, const float* xs, int64_t N, int32_t K, int32_t E,
                                int32_t d, int32_t d_ff, const int32_t* offsets,
                                const int32_t* sorted_slot, const uint8_t* w_gate,
                                const float* s_gate, const uint8_t* w_up, const float* s_up,
                                const uint8_t* w_down, const float* s_down, uint16_t* y_sorted,
                                void* workspace, size_t workspace_bytes, uint32_t flags,
                                void* stream);

/* ------------------------------------------------------------------------
 * Grouped SwiGLU experts of a top-1 dispatch (K = 1) with the weighted
 * combine done by the down projection's epilogue ("Mixture of experts" page,
 * Code: moe_infer's weighted sum, which for one choice per token is a scaled
 * copy back to token order; the same page's moe-init evidence: a GPU of an
 * expert-parallel group runs its local experts on rows it received, one
 * choice per row, and returns them in arrival order):
 *   out[n] = bfloat16( 0 + w[n] * y[n] ),  y[n] = the bfloat16 expert output
 * of token n as moe_grouped_swiglu computes it. The result equals
 * moe_grouped_swiglu followed by moe_combine (K = 1, no shared expert) bit for
 * bit, without the y_sorted round trip through memory.
 * x[N][d] bf16; offsets[E+1], sorted_slot[N] and slot_pos[N] from moe_dispatch
 * with K = 1; topk_w[N] float32; weights as moe_grouped_swiglu; out[N][d]
 * bf16, which must not overlap x. The workspace needs
 * moe_swiglu_workspace_size(N, 1, E, d, d_ff) bytes. Every out row is written
 * exactly once: a token whose id moe_dispatch left out (out of range, fast
 * mode: slot_pos[n] outside [0, N)) gets a +0 row, as moe_combine gives a
 * token with no valid choice. Shapes, alignment and flags as
 * moe_grouped_swiglu. N = 0 is a no-op.
 * ---------------------------------------------------------------------- */
moe_status moe_grouped_swiglu_top1(const uint16_t* x, int64_t N, int32_t E, int32_t d,
                                   int32_t d_ff, const int32_t* offsets,
                                   const int32_t* sorted_slot, const int32_t* slot_pos,
                                   const float* topk_w,
                                   const uint8_t* w_gate, const float* s_gate,
                                   const uint8_t* w_up, const float* s_up,
                                   const uint8_t* w_down, const float* s_down, uint16_t* out,
                                   void* workspace, size_t workspace_bytes, uint32_t flags,
                                   void* stream);

/* ------------------------------------------------------------------------
 * Weighted combine ("Mixture of experts" page, Code: moe_infer's weighted sum
 * over the K outputs of each token, and forward's addition of the shared
 * expert):
 *   out[n] = bfloat16( sum_{k=0..K-1} w[n][k] * y_sorted[slot_pos[n*K+k]]
 *                      + shared[n] )
 * summed in float32 in ascending k with the shared term last, one rounding to
 * bfloat16 (nearest-even). No atomics: deterministic.
 * y_sorted[N*K][d] bf16, slot_pos[N*K] int32 (from moe_dispatch; entries
 * outside [0, N*K) contribute nothing), topk_w[N][K] float32, shared[N][d] bf16
 * or NULL, out[N][d] bf16. d: positive multiple of 128. N = 0 is a no-op.
 * ---------------------------------------------------------------------- */
moe_status moe_combine(const uint16_t* y_sorted, const int32_t* slot_pos, const float* topk_w,
                       const uint16_t* shared, int64_t N, int32_t K, int32_t d, uint16_t* out,
                       void* stream);

/* The combine fused with the block's second residual addition ("Input
 * features" page, evidence "block": the FFN's output is added to the residual
 * stream it was computed from):
 *   out[n] = bfloat16( sum_k w[n][k] * y_sorted[slot_pos[n*K+k]] + shared[n]
 *                      + residual[n] )
 * in float32, in that order, one rounding. residual[N][d] bf16 is required;
 * out may be residual itself (the residual stream updated in place), but no
 * other overlap is allowed. Other arguments as moe_combine. */
moe_status moe_combine_residual(const uint16_t* y_sorted, const int32_t* slot_pos,
                                const float* topk_w, const uint16_t* shared,
                                const uint16_t* residual, int64_t N, int32_t K, int32_t d,
                                uint16_t* out, void* stream);

/* ------------------------------------------------------------------------
 * Dynamic e4m3 quantisation of bfloat16 rows, one float32 scale per 128
 * consecutive values ("Input features" page, evidence "linear": dynamic
 * activations, fmt e4m3): scale = amax/448 (1 for an all-zero group),
 * code = e4m3(value / scale) with IEEE division, nearest-even, saturating.
 * This is the first step of moe_grouped_swiglu, exported on its own.
 * x[rows][cols] bf16 -> q[rows][cols] e4m3, s[rows][cols/128] float32.
 * cols: positive multiple of 128, at most MOE_MAX_DIM; 0 <= rows < 2^31.
 * ---------------------------------------------------------------------- */
moe_status moe_quantize_rows(const uint16_t* x, int64_t rows, int32_t cols, uint8_t* q, float* s,
                             void* stream);

/* ------------------------------------------------------------------------
 * The block's RMSNorm before the FFN, fused with the quantisation of its
 * output ("Input features" page, evidence "rmsnorm": float32 normalisation,
 * returned in the input dtype and multiplied by the gain; evidence "linear"
 * for the e4m3 step). Per row of h[rows][cols] (bf16) with gain[cols] (bf16):
 *   v   = float32(mean of h_i^2)            (sum and division in double)
 *   r   = float32(1 / sqrt(float32(v + eps)))  (double, one rounding)
 *   y_i = bfloat16(gain_i * bfloat16(h_i * r))
 * then q, s = moe_quantize_rows(y) without storing y unless y is non-NULL
 * (y[rows][cols] bf16, for a router that reads the normalised features).
 * q and s feed moe_grouped_swiglu_q. cols: positive multiple of 128, at most
 * MOE_MAX_DIM; 0 <= rows < 2^31; eps >= 0 and finite. The squares of |h| above
 * about 1.8e19 would overflow float32 but not the double sum used here.
 * ---------------------------------------------------------------------- */
moe_status moe_rmsnorm_quantize_rows(const uint16_t* h, const uint16_t* gain, float eps,
                                     int64_t rows, int32_t cols, uint16_t* y, uint8_t* q,
                                     float* s, void* stream);

/* ------------------------------------------------------------------------
 * Diagnostics.
 * ---------------------------------------------------------------------- */
const char* moe_status_string(int status);
/* hipError_t value of the most recent MOE_ERR_HIP (0 if none), per thread. */
int moe_last_hip_error(void);

/* Per-kernel timing with HIP events recorded on the launch stream around each
 * launch of the library's kernels, for measuring the kernels inside a larger
 * timed region. Off by default. Kinds: MOE_KERNEL_*. moe_profile_read waits
 * for the recorded events, adds their elapsed times to the totals and returns
 * the totals since the last reset: summed milliseconds and launch count.
 * MOE_KERNEL_QUANT times the activation quantisation launch of moe_grouped_swiglu
 * and moe_grouped_swiglu_top1, which also builds the GEMM tile list;
 * MOE_KERNEL_DISPATCH times moe_dispatch and, in moe_grouped_swiglu_q, the tile
 * list's own launch. */
enum {
    MOE_KERNEL_QUANT = 0,
    MOE_KERNEL_DISPATCH = 1,
    MOE_KERNEL_GATE_UP = 2,
    MOE_KERNEL_DOWN = 3,
    MOE_KERNEL_COMBINE = 4,
    MOE_KERNEL_KINDS = 5
};
moe_status moe_profile_enable(int on);
/* Times only the kinds whose bit (1 << MOE_KERNEL_*) is set in kind_mask (0: none). Each timed
 * launch adds two event records to its stream, so a measurement that needs one kind's times
 * can leave the other launches uninstrumented. Bits above the last kind: MOE_ERR_SHAPE. */
moe_status moe_profile_enable_kinds(uint32_t kind_mask);
moe_status moe_profile_reset(void);
moe_status moe_profile_read(int kind, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
