/*
 * ds4moe.h - C ABI of libds4moe.so: the routed-MoE feed-forward block of ds4
 * (DeepSeek-V4-Flash) on one MI355X (gfx950), with 2-bit routed experts.
 *
 * The block, per token x (pages cited by title):
 *   - router: logits over all experts, softmax, top-k (lower expert index wins
 *     exact ties), weights renormalised over the k selected experts
 *     ("ds4 深度实战...", section 3.2 "MoE FFN": the router picks the experts;
 *     section 2.1: the router stays at full precision; "Redis 作者出手！ds4...",
 *     section 2.1: 256 routed experts, 6 used per token, 1 shared expert);
 *   - only the selected experts are computed ("ds4 深度实战...", section 3.2),
 *     each a SwiGLU feed-forward y = Wd (SiLU(Wg x) * (Wu x)) whose gate/up
 *     weights are IQ2-style 2-bit codebook blocks and whose down weights are
 *     Q2_K-style 2-bit blocks ("ds4 深度实战...", section 2.1; "Redis 作者出手！
 *     ds4...", section 2.3: 66-byte and 84-byte super-blocks of 256 weights);
 *   - the shared expert (bf16) runs on every token with weight 1 and its output
 *     is merged with the routed ones ("ds4 深度实战...", section 3.2);
 *   - the result is added into the caller's fp32 residual.
 *
 * Block formats (canonical, as the caller supplies them):
 *   IQ2-style, 66 bytes per 256 weights along the contraction dimension:
 *     bytes 0-1 fp16 d (little endian); 8 sub-blocks of 8 bytes, sub-block s
 *     covering weights 32s..32s+31 as 4 groups of 8: bytes 0-3 codebook
 *     indices of groups 0-3, bytes 4-7 a little-endian word with the signs of
 *     weights 0-6 of group g in bits 7g..7g+6 (1 = negative) and the sub-block
 *     scale ls in bits 28-31.  Weight 7's sign makes each group's count of
 *     negatives even.  Codebook entry: uint16, coordinate i in bits 2i..2i+1.
 *       w = d * (2 ls + 1)/8 * (2 c + 1)/8 * sign
 *   Q2_K-style, 84 bytes per 256 weights (field order of block_q2_K):
 *     scales[16] (low nibble sc, high nibble m, per 16 weights), qs[64]
 *     (weight i's 2-bit q at bits 2(i%4) of qs[i/4]), fp16 d, fp16 dmin.
 *       w = d * sc * q - dmin * m
 *
 * Conventions.  Pointers marked "device" are HIP device memory (for example
 * a torch tensor's data_ptr()), "host" are ordinary host memory.  `stream` is
 * a hipStream_t (NULL = the null stream).  Every call that takes a stream only
 * enqueues work on it: no host synchronisation and no allocation happen in
 * ds4moe_route / ds4moe_forward / ds4moe_dequantize / ds4moe_rmsnorm.
 *
 * Errors.  Every entry point returns DS4MOE_OK (0) or a negative status.
 * Arguments are validated before anything is enqueued; on a validation error
 * nothing is enqueued and ds4moe_last_error() describes it.  A HIP error
 * reported by a launch returns DS4MOE_EHIP and poisons the handle: later
 * calls on it return DS4MOE_EPOISONED.  No C++ exception crosses the ABI.
 *
 * Threading.  One handle serves one stream of calls at a time: calls on the
 * same handle must not overlap (they share the handle's workspace).  Distinct
 * handles are independent.
 */
#ifndef DS4MOE_H
#define DS4MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DS4MOE_ABI_VERSION 1

enum {
    DS4MOE_OK = 0,
    DS4MOE_EINVAL = -1,       /* bad argument; nothing enqueued */
    DS4MOE_ENOMEM = -2,       /* device allocation failed in ds4moe_create */
    DS4MOE_EHIP = -3,         /* a HIP call failed; the handle is poisoned */
    DS4MOE_EUNSUPPORTED = -4, /* valid but unsupported combination */
    DS4MOE_EPOISONED = -5     /* handle unusable after an earlier HIP error */
};

enum { DS4MOE_F32 = 0, DS4MOE_BF16 = 1 };

/* Kernel path selection for ds4moe_forward (ds4moe_set_path). */
enum {
    DS4MOE_PATH_AUTO = 0,    /* one token: fused decode; 2-4 fp32 tokens: GEMV; else grouped MFMA GEMM */
    DS4MOE_PATH_GEMV = 1,    /* dequant-fused GEMV kernels (decode); n_tok <= 4 only,
                                else ds4moe_forward returns DS4MOE_EUNSUPPORTED */
    DS4MOE_PATH_GEMM = 2     /* grouped dequant MFMA GEMM kernels (prefill), any n_tok */
};

typedef struct ds4moe ds4moe_t; /* opaque; one per MoE layer */

/*
 * Layer description passed to ds4moe_create.
 *   n_embd, n_ff: each one of 256, 512, 1024, 2048, 4096 (whole super-blocks of 256
 *                 weights; one 128-bit load per lane covers 64 weights of a row).
 *   n_expert in 1..256; top_k in 1..min(n_expert, 8); n_shared 0 or 1.
 *   max_tokens >= 1: the largest n_tok later passed to route/forward (sizes the workspace).
 *   act_dtype: DS4MOE_F32 or DS4MOE_BF16, the element type of x.
 *   router:      device, fp32 [n_expert][n_embd] (expert-major).
 *   router_bias: device, fp32 [n_expert], or NULL (added to the logits before the softmax).
 *   gate, up:    device, IQ2-style blocks [n_expert][n_ff][n_embd/256][66 bytes].
 *   down:        device, Q2_K-style blocks [n_expert][n_embd][n_ff/256][84 bytes].
 *   codebook:    host, uint16 [256].
 *   sh_gate, sh_up: device, bf16 [n_ff][n_embd]; sh_down: device, bf16 [n_embd][n_ff];
 *                all NULL when n_shared == 0.
 */
typedef struct {
    int32_t abi_version; /* DS4MOE_ABI_VERSION */
    int32_t n_embd, n_ff, n_expert, top_k, n_shared, max_tokens, act_dtype;
    const float *router;
    const float *router_bias;
    const void *gate;
    const void *up;
    const void *down;
    const uint16_t *codebook;
    const uint16_t *sh_gate;
    const uint16_t *sh_up;
    const uint16_t *sh_down;
} ds4moe_desc;

/*
 * Create a layer handle.  Reads the caller's weights on `stream`, repacks the
 * routed experts into the library's own device layout (same bytes per weight,
 * planes aligned for 128-bit loads), copies the router and shared expert,
 * allocates the workspace for max_tokens, synchronises `stream` and returns.
 * The caller may free its weight buffers afterwards.  *out is set only on
 * success.  Errors: EINVAL (bad description), ENOMEM, EHIP.
 */
int ds4moe_create(const ds4moe_desc *desc, void *stream, ds4moe_t **out);

/*
 * Router and token bucketing only (the front of ds4moe_forward), with the
 * results exposed.  x: device [n_tok][n_embd] of act_dtype.  Outputs, device:
 *   topk_idx [n_tok][top_k] int32: selected experts, slot order = decreasing
 *            logit, lower index first among equal logits;
 *   topk_w   [n_tok][top_k] fp32: softmax probabilities renormalised over the
 *            selected experts;
 *   expert_offsets [n_expert+1] int32 and expert_tokens [n_tok*top_k] int32:
 *            expert e's tokens are expert_tokens[offsets[e] .. offsets[e+1]),
 *            in ascending token order.
 * Logits are accumulated in fp64 and rounded to fp32 before selection.
 * 0 <= n_tok <= max_tokens; n_tok == 0 enqueues nothing (outputs untouched).
 */
int ds4moe_route(ds4moe_t *h, const void *x, int32_t n_tok, int32_t *topk_idx, float *topk_w,
                 int32_t *expert_offsets, int32_t *expert_tokens, void *stream);

/*
 * out += MoE(x): x device [n_tok][n_embd] of act_dtype; out device fp32
 * [n_tok][n_embd], read and written (pass zeros for the bare block output).
 * 0 <= n_tok <= max_tokens; n_tok == 0 is a no-op.  x and out must not overlap;
 * both 16-byte aligned.  The routed and shared contributions are added with
 * fp32 atomics, so the summation order (last bits) may vary between runs.
 */
int ds4moe_forward(ds4moe_t *h, const void *x, int32_t n_tok, float *out, void *stream);

/* Choose the kernel path used by ds4moe_forward (DS4MOE_PATH_*).  Host-only. */
int ds4moe_set_path(ds4moe_t *h, int32_t path);

/*
 * Debug/test: decode one routed expert matrix from the library's repacked
 * layout.  which: 0 gate, 1 up ([n_ff][n_embd] fp32), 2 down ([n_embd][n_ff]
 * fp32).  dst: device, fp32, that many elements.
 */
int ds4moe_dequantize(ds4moe_t *h, int32_t expert, int32_t which, float *dst, void *stream);

/*
 * RMSNorm with unit gain between stacked layers:
 *   x_bf16[t][i] = bf16_rne( h[t][i] / sqrt(mean_i h[t][i]^2 + eps) )
 * computed in fp64.  h: device fp32 [n_tok][n_embd]; x_bf16: device bf16 bits.
 * n_tok >= 0, 1 <= n_embd <= 65536, eps >= 0.
 */
int ds4moe_rmsnorm(const float *h, int32_t n_tok, int32_t n_embd, double eps, uint16_t *x_bf16,
                   void *stream);

/*
 * A stack of layers on one residual stream: the per-layer loop of the
 * inference pseudo-code ("ds4 深度实战...", section 3.2) with attention left
 * out and a unit-gain RMSNorm in front of each MoE block.  For
 * l = 0 .. n_layers-1,
 *   x = RMSNorm(h)  (exactly as ds4moe_rmsnorm with eps), then
 *   h += MoE_l(x)   (exactly as ds4moe_forward on layers[l]).
 * h: device fp32 [n_tok][n_embd], updated in place.  x_bf16: device scratch
 * of n_tok * n_embd bf16 values, caller-owned, overwritten.  Every layer must
 * take bf16 activations, share n_embd and allow n_tok tokens.  All launches
 * are enqueued from this one host call (two per layer at n_tok = 1), so the
 * host does not pace the device.  Errors: every layer is validated before
 * anything is enqueued (DS4MOE_EINVAL / DS4MOE_EPOISONED, nothing enqueued);
 * a launch failure at layer l returns DS4MOE_EHIP with layers before l
 * already enqueued, and the message names l.
 */
int ds4moe_forward_stack(ds4moe_t *const *layers, int32_t n_layers, float *h, int32_t n_tok, double eps,
                         uint16_t *x_bf16, void *stream);

/*
 * Per-kernel timing for benchmarks.  When enabled, ds4moe_forward records HIP
 * events around each kernel it launches on the caller's stream; read back the
 * accumulated milliseconds and launch counts (after synchronising the stream)
 * with ds4moe_timing_read.  kinds: 0 route (logits, top-k, lists), 1 routed
 * gate/up GEMV, 2 shared gate/up GEMV, 3 routed down GEMV, 4 shared down GEMV,
 * 5 routed gate/up GEMM, 6 routed down GEMM, 7 fused decode kernel, 8 batched
 * path preparation (activation copies, chunk table), 9 shared gate/up GEMM,
 * 10 shared down GEMM.  ms and counts have room for DS4MOE_TIMING_KINDS
 * entries each.  Enabling resets the counters.
 */
#define DS4MOE_TIMING_KINDS 11
int ds4moe_timing_enable(ds4moe_t *h, int32_t enable);
int ds4moe_timing_read(ds4moe_t *h, double *ms, int64_t *counts);

/* Free everything the handle owns (after the caller's stream work is done).  NULL is a no-op. */
int ds4moe_destroy(ds4moe_t *h);

/* Message for the last error on the calling thread ("" if none). */
const char *ds4moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DS4MOE_H */
