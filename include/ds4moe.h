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
 * ds4moe_route / ds4moe_forward / ds4moe_dequantize / ds4moe_rmsnorm.  A
 * forward call on a bf16 layer with a shared expert that takes the grouped
 * path (more tokens than the small-batch kernels take) runs the shared expert
 * on a second stream of the handle (created with it): forked from `stream`
 * by an event, and joined back into `stream` within the call, so that all of
 * the call's work is ordered before whatever is enqueued on `stream` after it.
 *
 * Errors.  Every entry point returns DS4MOE_OK (0) or a negative status.
 * Arguments are validated before anything is enqueued; on a validation error
 * nothing is enqueued and ds4moe_last_error() describes it.  A HIP error
 * reported by a launch returns DS4MOE_EHIP and poisons the handle: later
 * calls on it return DS4MOE_EPOISONED.  Kernels that hand data between
 * workgroups bound every wait; a wait that gives up writes NaN into the
 * call's output and records the call in a host-visible status word of the
 * handle, so the next call on the handle (or ds4moe_status) returns
 * DS4MOE_EPOISONED without any host synchronisation.  No C++ exception
 * crosses the ABI.
 *
 * Threading.  One handle serves one stream of calls at a time: calls on the
 * same handle must not overlap (they share the handle's workspace).  Distinct
 * handles are independent.
 *
 * Graph capture.  The hand-offs between workgroups are tagged with host-side
 * call counts, which a captured graph would replay unchanged: route, forward,
 * forward_stack and last_routing refuse a stream that is being captured
 * (DS4MOE_EUNSUPPORTED, nothing enqueued).
 */
#ifndef DS4MOE_H
#define DS4MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DS4MOE_ABI_VERSION 4

enum {
    DS4MOE_OK = 0,
    DS4MOE_EINVAL = -1,       /* bad argument; nothing enqueued */
    DS4MOE_ENOMEM = -2,       /* device allocation failed in ds4moe_create */
    DS4MOE_EHIP = -3,         /* a HIP call failed; the handle is poisoned */
    DS4MOE_EUNSUPPORTED = -4, /* valid but unsupported combination */
    DS4MOE_EPOISONED = -5     /* handle unusable after an earlier HIP error, an expired
                                 bounded wait or a token id out of range */
};

enum { DS4MOE_F32 = 0, DS4MOE_BF16 = 1 };

/* Routed-expert block formats (ds4moe_desc.expert_format). */
enum {
    DS4MOE_FMT_Q2 = 0, /* gate/up IQ2-style (66 B / 256 weights), down Q2_K-style (84 B) */
    DS4MOE_FMT_Q4 = 1  /* gate, up and down Q4_K-style (144 B / 256 weights) */
};

/* Kernel path selection for ds4moe_forward (ds4moe_set_path). */
enum {
    DS4MOE_PATH_AUTO = 0,    /* one token: fused decode; 2-4 fp32 tokens: GEMV; 2..DS4MOE_SMALL_MAX_TOKENS
                                bf16 tokens on a layer that has it: small-batch kernels; else grouped MFMA GEMM */
    DS4MOE_PATH_GEMV = 1,    /* dequant-fused GEMV kernels (decode); n_tok <= 4 only,
                                else ds4moe_forward returns DS4MOE_EUNSUPPORTED */
    DS4MOE_PATH_GEMM = 2,    /* grouped dequant MFMA GEMM kernels (prefill), any n_tok */
    DS4MOE_PATH_SMALL = 3    /* small-batch kernels: the router, then two persistent MFMA launches that
                                stream each selected expert once for all of its tokens (speculative
                                verification batches, "ds4 深度实战...", sections 4.2 and 4.4).  Layers
                                with bf16 activations, the 2-bit format, n_ff <= 2048 and max_tokens >= 2
                                (else ds4moe_set_path returns DS4MOE_EUNSUPPORTED); ds4moe_forward takes
                                2..DS4MOE_SMALL_MAX_TOKENS tokens on it (else DS4MOE_EUNSUPPORTED) */
};
#define DS4MOE_SMALL_MAX_TOKENS 8

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
 *   expert_format: DS4MOE_FMT_Q2 (the layouts above) or DS4MOE_FMT_Q4: gate, up
 *                and down are all Q4_K-style blocks, [n_expert][rows][cols/256][144
 *                bytes]: fp16 d, fp16 dmin, sixteen 6-bit fields as a little-
 *                endian bit stream (field j at bits 6j..6j+5: sc of sub-block j
 *                for j < 8, m of sub-block j-8 for j >= 8; sub-block = 32 weights),
 *                then 128 bytes of 4-bit quants (weight i in nibble i%2 of byte
 *                i/2, low nibble first); w = d sc q - dmin m.  The q4 model keeps
 *                its routed experts in Q4_K ("ds4 深度实战...", section 2.1; the
 *                pages give no layout: this one is a stand-in).  codebook is
 *                unused.  A q4 layer runs the dequant-fused GEMV kernels for
 *                every call, in chunks of up to 4 tokens.
 *   hash_table, n_vocab: a hash-routed layer (the model's hash layers,
 *                DS4_N_HASH_LAYER = 3 in the model constants of "Redis 作者出手！
 *                ds4...", section 2.1; the pages say nothing more, so this is a
 *                reading): token t's experts are row token_ids[t] of the table,
 *                in slot order, and their weights are the router's softmax
 *                renormalised over them.  Each row must hold top_k distinct
 *                experts in 0..n_expert-1 (checked at create: EINVAL); 1 <=
 *                n_vocab <= INT32_MAX / top_k; 4-byte aligned.  The table is
 *                copied.  Such a layer is called through the *_ids entry points.
 *   expert_cache_slots: 0 keeps every routed expert in HBM.  S in top_k..n_expert
 *                keeps the routed experts in pinned host memory (copied there at
 *                create, in the library's layout) and S of them in HBM: the
 *                model's way to run when it does not fit in GPU memory, with the
 *                non-routed weights resident and a routed expert loaded on a
 *                miss ("DS-4 DwarfStar - DeepSeek V4 Flash 本地推理引擎", section
 *                "SSD Streaming", how it works; "ds4 深度实战...", section 3.5).
 *                Each call routes, then one workgroup updates the cache (the
 *                call's resident experts are stamped, each missing expert takes
 *                a slot the call does not use: empty ones first, then the least
 *                recently used, lower slot first on equal stamps) and a copy
 *                kernel pulls the missed experts over the host link into their
 *                slots, all on the call's stream with no host synchronisation;
 *                the expert kernels then read each expert at its slot.  A call
 *                is run in sub-calls of at most S / top_k tokens (unless S ==
 *                n_expert), so that its distinct experts fit; one token runs on
 *                the GEMV kernels instead of the fused decode kernel.  The
 *                results equal those of a layer with every expert in HBM.
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
    int32_t expert_format; /* DS4MOE_FMT_Q2 or DS4MOE_FMT_Q4 */
    const int32_t *hash_table; /* device int32 [n_vocab][top_k], or NULL (learned routing) */
    int64_t n_vocab;           /* rows of hash_table (ignored when it is NULL) */
    int32_t expert_cache_slots; /* 0: every routed expert in HBM; else host-resident experts, this many in HBM */
} ds4moe_desc;

/*
 * Create a layer handle: one routed-MoE layer with 256 (n_expert) routed
 * experts, top-k routing and one shared expert ("Redis 作者出手！ds4...",
 * section 2.1, the model constants; section 2.3, the two 2-bit block formats
 * and the high-precision shared expert).  Reads the caller's weights on `stream`, repacks the
 * routed experts into the library's own device layout (same bytes per weight,
 * planes aligned for 128-bit loads), copies the router and shared expert,
 * allocates the workspace for max_tokens, synchronises `stream` and returns.
 * The caller may free its weight buffers afterwards.  *out is set only on
 * success.  Errors: EINVAL (bad description), ENOMEM, EHIP.
 */
int ds4moe_create(const ds4moe_desc *desc, void *stream, ds4moe_t **out);

/*
 * Router and token bucketing only (the front of ds4moe_forward), with the
 * results exposed.  The router scores every expert and only the chosen ones
 * are computed ("ds4 深度实战...", section 3.2 "MoE FFN"; section 3.3: experts
 * are scheduled from the router's output); 6 of 256 per token ("Redis 作者出
 * 手！ds4...", section 2.1).  The gating is softmax, top-k and renormalisation
 * over the selected experts.  x: device [n_tok][n_embd] of act_dtype.  Outputs, device:
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
 * ds4moe_route with the tokens' ids, for a hash-routed layer (the model's
 * hash layers: "Redis 作者出手！ds4...", section 2.1, DS4_N_HASH_LAYER).
 * token_ids: device int32 [n_tok], 4-byte aligned, each in 0..n_vocab-1;
 * ignored (may be NULL) for a learned-routing layer, which it routes exactly
 * as ds4moe_route.  On a hash layer topk_idx[t] is the table's row
 * token_ids[t] in slot order and topk_w[t] the softmax over all logits
 * renormalised over those experts, which depends on their k logits alone
 * (only those k router rows are read).  An id out of range cannot be seen
 * without synchronising: that token's weights (and its block output) become
 * NaN, and the handle reports DS4MOE_EPOISONED from its next call on.  The
 * plain entry points (route, forward, forward_stack) refuse a hash layer
 * with DS4MOE_EINVAL, and ds4moe_forward_static with DS4MOE_EUNSUPPORTED.
 */
int ds4moe_route_ids(ds4moe_t *h, const void *x, const int32_t *token_ids, int32_t n_tok, int32_t *topk_idx,
                     float *topk_w, int32_t *expert_offsets, int32_t *expert_tokens, void *stream);

/*
 * The block ("ds4 深度实战...", section 3.2 "MoE FFN": route, compute only the
 * chosen experts and the shared expert, merge their outputs; section 2.1: the
 * routed gate/up in IQ2_XXS, down in Q2_K, shared expert at full precision).
 * out += MoE(x): x device [n_tok][n_embd] of act_dtype; out device fp32
 * [n_tok][n_embd], read and written (pass zeros for the bare block output).
 * 0 <= n_tok <= max_tokens; n_tok == 0 is a no-op.  x and out must not overlap;
 * both 16-byte aligned.  The routed and shared contributions are added with
 * fp32 atomics, so the summation order (last bits) may vary between runs.
 */
int ds4moe_forward(ds4moe_t *h, const void *x, int32_t n_tok, float *out, void *stream);

/*
 * ds4moe_forward with the tokens' ids (token_ids as for ds4moe_route_ids):
 * the block of a hash-routed layer, with the same kernels as ds4moe_forward
 * after the routing; a learned-routing layer ignores the ids.
 */
int ds4moe_forward_ids(ds4moe_t *h, const void *x, const int32_t *token_ids, int32_t n_tok, float *out,
                       void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture elsewhere in their program, tight serving loops, harnesses that
 * forbid hipMalloc): out += MoE(x) for 1 <= n_tok <= DS4MOE_STATIC_MAX_TOKENS
 * tokens, with the results of ds4moe_forward on the same inputs (one token:
 * the fused decode kernel; 2..4: the dequant-fused GEMV kernels, whatever
 * ds4moe_set_path says), but every scratch buffer of the call (routing
 * results, tagged hand-off words, the router's tickets, SwiGLU activations)
 * in the library's static device array of DS4MOE_STATIC_SCRATCH_BYTES, one
 * per GPU, which each GPU holds until the process ends; the handle's own
 * workspace is not touched.  Nothing is allocated.  The handle's device must
 * be current.  n_tok > DS4MOE_STATIC_MAX_TOKENS returns DS4MOE_EINVAL
 * (nothing enqueued); n_tok == 0 is a no-op.  Calls on one GPU share its
 * array: calls that overlap on one GPU (on any handles, on different streams)
 * race and must be serialised by the caller; consecutive stream-ordered calls
 * are safe (their hand-off tags come from one per-GPU count).  x, out and the
 * errors are as for ds4moe_forward; a stream under capture is refused.
 */
#define DS4MOE_STATIC_SCRATCH_BYTES (1u << 20)
#define DS4MOE_STATIC_MAX_TOKENS 4
int ds4moe_forward_static(ds4moe_t *h, const void *x, int32_t n_tok, float *out, void *stream);

/* Choose the kernel path used by ds4moe_forward (DS4MOE_PATH_*).  Host-only. */
int ds4moe_set_path(ds4moe_t *h, int32_t path);

/*
 * Debug/test: decode one routed expert matrix from the library's repacked
 * layout ("Redis 作者出手！ds4...", section 2.3: block_iq2_xxs for gate/up,
 * block_q2_K for down, each 256 weights per super-block; Q4_K-style for all
 * three in a q4 layer).  which: 0 gate, 1 up ([n_ff][n_embd] fp32), 2 down ([n_embd][n_ff]
 * fp32).  dst: device, fp32, that many elements.
 */
int ds4moe_dequantize(ds4moe_t *h, int32_t expert, int32_t which, float *dst, void *stream);

/*
 * Debug/test: one routed expert matrix exactly as the grouped GEMM kernels
 * feed it to the MFMAs, each fp16 value widened to fp32, through the same
 * device code (which and dst as for ds4moe_dequantize).  The 2-bit weights
 * are rounded to fp16 there: an IQ2 weight is its signed level times
 * fp16(d (2 ls + 1) / 64), rounded again in the product; a Q2_K weight is
 * fma(q, fp16(d sc), fp16(-dmin m)) in fp16.  IQ2 values are decoded twice,
 * with the signs from bit arithmetic and from the sign-mask table (the two
 * decodes the kernels use); a value on which they differ in any bit is
 * written as NaN.  DS4MOE_EUNSUPPORTED for a q4 layer (its kernels form no
 * rounded weight: the 4-bit codes enter fp16 dot products exactly, as
 * 1 + q/64, and d sc and dmin m are applied in fp32 per sub-block).
 */
int ds4moe_debug_gemm_b(ds4moe_t *h, int32_t expert, int32_t which, float *dst, void *stream);

/*
 * RMSNorm with unit gain between stacked layers (the stack of 43 layers,
 * "Redis 作者出手！ds4...", section 2.1; the pages' model mixes layers through
 * hyper-connections instead, which this block leaves out):
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
 * ds4moe_forward_stack with the tokens' ids, for stacks holding hash-routed
 * layers (the model's first layers; "Redis 作者出手！ds4...", section 2.1,
 * DS4_N_HASH_LAYER = 3): every layer runs as ds4moe_forward_ids with the same
 * token_ids (device int32 [n_tok]); NULL is allowed when no layer hashes.
 */
int ds4moe_forward_stack_ids(ds4moe_t *const *layers, int32_t n_layers, float *h, const int32_t *token_ids,
                             int32_t n_tok, double eps, uint16_t *x_bf16, void *stream);

/*
 * The HBM expert cache of a layer created with expert_cache_slots > 0
 * (DS4MOE_EUNSUPPORTED otherwise).  ds4moe_cache_stats writes, to host
 * stats[4]: calls (sub-calls) so far, expert hits, expert misses, and bytes
 * copied from host memory.  ds4moe_cache_slots writes, to host
 * slot_expert[expert_cache_slots], the expert each slot holds (-1: empty).
 * Both enqueue a copy on `stream` and synchronise it.
 */
int ds4moe_cache_stats(ds4moe_t *h, int64_t *stats, void *stream);
int ds4moe_cache_slots(ds4moe_t *h, int32_t *slot_expert, void *stream);

/*
 * Per-kernel timing for benchmarks.  When enabled, ds4moe_forward records HIP
 * events around each kernel it launches on the caller's stream; read back the
 * accumulated milliseconds and launch counts (after synchronising the stream)
 * with ds4moe_timing_read.  kinds: 0 route (logits, top-k, lists), 1 routed
 * gate/up GEMV, 2 shared gate/up GEMV, 3 routed down GEMV, 4 shared down GEMV,
 * 5 routed gate/up GEMM, 6 routed down GEMM, 7 fused decode kernel, 8 batched
 * path preparation (activation copies, chunk table), 9 shared gate/up GEMM,
 * 10 shared down GEMM, 11 routed gate/up Q4_K GEMV, 12 routed down Q4_K
 * GEMV, 13 expert cache update and copy, 14 small-batch gate/up kernel, 15
 * small-batch down kernel.  ms and counts have room for DS4MOE_TIMING_KINDS entries each.
 * Enabling resets the counters.
 */
#define DS4MOE_TIMING_KINDS 16
int ds4moe_timing_enable(ds4moe_t *h, int32_t enable);
int ds4moe_timing_read(ds4moe_t *h, double *ms, int64_t *counts);

/*
 * The routing that the most recent ds4moe_forward or ds4moe_route call on h
 * computed (for a one-token forward, the fused decode kernel's own top-k),
 * copied into the caller's device buffers with the layouts of ds4moe_route.
 * n_tok must equal that call's n_tok (EINVAL otherwise).  Stream-ordered
 * after that call.  The same selection rule as ds4moe_route ("ds4 深度实战...",
 * section 3.2).
 */
int ds4moe_last_routing(ds4moe_t *h, int32_t n_tok, int32_t *topk_idx, float *topk_w, int32_t *expert_offsets,
                        int32_t *expert_tokens, void *stream);

/*
 * DS4MOE_OK, or DS4MOE_EPOISONED (the handle is then poisoned) if a bounded
 * wait of an earlier call on h gave up or a HIP error poisoned it.  Reads the
 * host-visible status word only: synchronise the stream first for a
 * definitive answer about calls still in flight.
 */
int ds4moe_status(ds4moe_t *h);

/*
 * Test hook for the bounded waits of h's kernels: max_polls is the number of
 * polls before a wait gives up (0 restores the default, about a second), and
 * force_expire != 0 makes every wait look for a tag that no producer writes,
 * so every wait gives up after max_polls polls while every kernel still runs
 * to its end.  Host-only.
 */
int ds4moe_set_wait_limit(ds4moe_t *h, int32_t max_polls, int32_t force_expire);

/* Free everything the handle owns (after the caller's stream work is done).  NULL is a no-op. */
int ds4moe_destroy(ds4moe_t *h);

/* Message for the last error on the calling thread ("" if none). */
const char *ds4moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DS4MOE_H */
