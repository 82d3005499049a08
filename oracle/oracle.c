/*
 * oracle.c - plain, slow CPU oracle for ds4's 2-bit routed-MoE feed-forward block.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  It shares no code,
 * header, table or helper with the HIP library, and the HIP library never
 * calls it.
 *
 * What it computes (every function below cites the passage it follows):
 *
 *  - the routed-expert block formats (IQ2-style gate/up with Q2_K-style down,
 *    or Q4_K-style for all three), decoded one weight at a time into fp32
 *    (every decoded value is exact in fp32 for the value ranges used);
 *  - the router: fp64-accumulated logits rounded to fp32, a softmax over all
 *    experts, the top-k experts (lower index wins exact ties) and the weights
 *    renormalised over the selected experts;
 *  - hash routing for the model's hash layers: the experts looked up from a
 *    per-token-id table, the weights the router's softmax renormalised over
 *    them (the pages give only the layer count; this is the reading used);
 *  - per-expert token lists (ascending token order);
 *  - the block output: for each token, the weighted sum of its selected
 *    experts' SwiGLU feed-forward outputs plus the shared expert's output,
 *    every matmul accumulated in fp64 with one accumulator, in index order;
 *  - the RMSNorm used between stacked layers.
 *
 * Citations name the pages by title:
 *   [P1] "ds4 深度实战：当 Redis 之父用纯 C 重写本地推理引擎..."
 *   [P2] "DS-4 DwarfStar - DeepSeek V4 Flash 本地推理引擎"
 *   [P5] "Redis 作者出手！ds4：用 C 语言从零打造 DeepSeek V4 Flash 本地推理引擎..."
 * The pages name IQ2_XXS and Q2_K and print only their struct sizes; the bit
 * layouts, the codebook and the gating function are the stand-in formats and
 * readings fixed for this block (listed in the repository's design notes).
 *
 * Every function is pinned by tests that do not retype its formula:
 * round trips through an independent encoder, structural invariants, brute
 * force on tiny inputs and textbook dense SwiGLU via numpy matmuls.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QK 256

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t rd32(const uint8_t *p)
{
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

/* IEEE binary16 -> double, exact. */
static double half_value(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);
    return sign ? -v : v;
}

/* bfloat16 bit pattern -> double, exact. */
static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* double -> bfloat16 bits, round to nearest, ties to even (normal range). */
static uint16_t bf16_round(double v)
{
    if (v == 0.0 || !isfinite(v)) {
        float f = (float)v;
        uint32_t u;
        memcpy(&u, &f, 4);
        return (uint16_t)(u >> 16);
    }
    int e;
    double m = frexp(fabs(v), &e);          /* |v| = m * 2^e, m in [0.5, 1) */
    double r = nearbyint(ldexp(m, 8));      /* 8 significant bits, ties to even */
    float f = (float)ldexp(v < 0 ? -r : r, e - 8);
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static int popcount7(uint32_t v)
{
    int n = 0;
    for (int i = 0; i < 7; ++i)
        n += (v >> i) & 1;
    return n;
}

/*
 * IQ2-style super-block, 66 bytes per 256 weights ([P5] section 2.3 gives the
 * size: one fp16 d plus 32 uint16 of quant data; [P1] section 2.1 and [P5]
 * section 2.3 put the routed gate/up projections in this format).
 *
 * Layout: bytes 0-1 fp16 d; then 8 sub-blocks of 8 bytes, sub-block s holding
 * weights 32s..32s+31 as 4 groups of 8.  In a sub-block, bytes 0-3 are the
 * codebook indices of groups 0-3 and bytes 4-7 a little-endian word whose bits
 * 7g..7g+6 are the signs of weights 0-6 of group g (1 = negative) and whose
 * bits 28-31 are the sub-block scale ls.  Weight 7 of a group is negative when
 * the other seven signs hold an odd number of negatives, so each group has an
 * even number of negative weights.  Codebook entry coordinate i (bits 2i..2i+1)
 * is c in 0..3, magnitude (2c+1)/8.
 *
 *   w = d * (2 ls + 1)/8 * (2 c + 1)/8 * sign
 */
void oracle_dequant_iq2(const uint8_t *blocks, int64_t n_blocks, const uint16_t *codebook, float *out)
{
    for (int64_t b = 0; b < n_blocks; ++b) {
        const uint8_t *blk = blocks + 66 * b;
        double d = half_value(rd16(blk));
        for (int s = 0; s < 8; ++s) {
            const uint8_t *sub = blk + 2 + 8 * s;
            uint32_t word = rd32(sub + 4);
            int ls = (int)(word >> 28);
            double sub_scale = (2.0 * ls + 1.0) / 8.0;
            for (int g = 0; g < 4; ++g) {
                uint16_t entry = codebook[sub[g]];
                uint32_t signs = (word >> (7 * g)) & 0x7F;
                int odd = popcount7(signs) & 1;
                for (int i = 0; i < 8; ++i) {
                    int c = (entry >> (2 * i)) & 3;
                    int negative = (i < 7) ? (int)((signs >> i) & 1) : odd;
                    double v = d * sub_scale * ((2.0 * c + 1.0) / 8.0);
                    out[QK * b + 32 * s + 8 * g + i] = (float)(negative ? -v : v);
                }
            }
        }
    }
}

/*
 * Q2_K-style super-block, 84 bytes per 256 weights.  Field order from the
 * block_q2_K struct on [P5] section 2.3: scales[16], qs[64], fp16 d, fp16 dmin
 * ([P1] section 2.1: the routed down projection uses it).
 *
 * scales[s]: low nibble sc, high nibble m, for weights 16s..16s+15.
 * qs: weight i's 2-bit quant q is bits 2(i%4)..2(i%4)+1 of qs[i/4].
 *
 *   w = d * sc * q - dmin * m
 */
void oracle_dequant_q2k(const uint8_t *blocks, int64_t n_blocks, float *out)
{
    for (int64_t b = 0; b < n_blocks; ++b) {
        const uint8_t *blk = blocks + 84 * b;
        double d = half_value(rd16(blk + 80));
        double dmin = half_value(rd16(blk + 82));
        for (int i = 0; i < QK; ++i) {
            int s = i / 16;
            int sc = blk[s] & 15;
            int m = blk[s] >> 4;
            int q = (blk[16 + i / 4] >> (2 * (i % 4))) & 3;
            out[QK * b + i] = (float)(d * sc * q - dmin * m);
        }
    }
}

/*
 * Q4_K-style super-block, 144 bytes per 256 weights: the routed experts of the
 * q4 model ([P1] section 2.1: the q2-q4 variant keeps its last 6 layers at q4;
 * [P5] section 3.1 names the format Q4 (Q4_K)).  The pages give no layout, so
 * the packing is the stand-in fixed for this block:
 *   bytes 0-1 fp16 d, bytes 2-3 fp16 dmin (little endian);
 *   bytes 4-15 a little-endian stream of sixteen 6-bit fields, field j at
 *   stream bits 6j..6j+5: for j < 8 the scale sc of sub-block j (weights
 *   32j..32j+31), for j >= 8 the min m of sub-block j-8;
 *   bytes 16-143 the 4-bit quants: weight i's q is bits 4(i%2)..4(i%2)+3 of
 *   byte 16 + i/2.
 *   w = d * sc * q - dmin * m
 */
static int q4k_field(const uint8_t *blk, int j)
{
    int v = 0;
    for (int b = 0; b < 6; ++b) {
        int bit = 6 * j + b;
        v |= ((blk[4 + bit / 8] >> (bit % 8)) & 1) << b;
    }
    return v;
}

void oracle_dequant_q4k(const uint8_t *blocks, int64_t n_blocks, float *out)
{
    for (int64_t b = 0; b < n_blocks; ++b) {
        const uint8_t *blk = blocks + 144 * b;
        double d = half_value(rd16(blk));
        double dmin = half_value(rd16(blk + 2));
        for (int i = 0; i < QK; ++i) {
            int s = i / 32;
            int sc = q4k_field(blk, s);
            int m = q4k_field(blk, 8 + s);
            int q = (blk[16 + i / 2] >> (4 * (i % 2))) & 15;
            out[QK * b + i] = (float)(d * sc * q - dmin * m);
        }
    }
}

static double x_value(const void *x, int x_is_bf16, int64_t i)
{
    return x_is_bf16 ? bf16_value(((const uint16_t *)x)[i]) : (double)((const float *)x)[i];
}

/*
 * Router for one token ([P1] section 3.2: the router chooses the experts and
 * only those are computed; [P1] section 2.1 and [P2] keep the router at full
 * precision; [P5] section 2.1: 6 of 256 experts per token).
 *
 * 1. logits L[e] = fp32( sum_i x[i] R[e][i] + bias[e] ), summed in fp64;
 * 2. softmax over all experts: p[e] = exp(L[e] - max L) / sum exp(L - max L);
 * 3. top-k: experts in decreasing p, lower index first among equals.  p is a
 *    strictly increasing function of L, so the order is taken on the exact
 *    fp32 logits (rounding of p cannot create false ties);
 * 4. renormalise: w[j] = p[sel j] / sum_j p[sel j].
 * Slots are emitted in selection order.  Weights are returned in fp64.
 */
static void route_token(const double *xt, int n_embd, const float *router, const float *bias,
                        int n_expert, int top_k, float *logits, double *p, int32_t *idx, double *w)
{
    for (int e = 0; e < n_expert; ++e) {
        double s = 0.0;
        const float *r = router + (int64_t)e * n_embd;
        for (int i = 0; i < n_embd; ++i)
            s += xt[i] * (double)r[i];
        if (bias)
            s += (double)bias[e];
        logits[e] = (float)s;
    }
    double mx = -INFINITY;
    for (int e = 0; e < n_expert; ++e)
        if ((double)logits[e] > mx)
            mx = logits[e];
    double z = 0.0;
    for (int e = 0; e < n_expert; ++e) {
        p[e] = exp((double)logits[e] - mx);
        z += p[e];
    }
    for (int e = 0; e < n_expert; ++e)
        p[e] /= z;

    for (int j = 0; j < top_k; ++j) {
        int best = -1;
        for (int e = 0; e < n_expert; ++e) {
            int taken = 0;
            for (int q = 0; q < j; ++q)
                taken |= idx[q] == e;
            if (taken)
                continue;
            if (best < 0 || logits[e] > logits[best])
                best = e;
        }
        idx[j] = best;
    }
    double sum = 0.0;
    for (int j = 0; j < top_k; ++j)
        sum += p[idx[j]];
    for (int j = 0; j < top_k; ++j)
        w[j] = p[idx[j]] / sum;
}

/*
 * Hash routing ([P5] section 2.1: DS4_N_HASH_LAYER = 3, the model's hash
 * layers; the pages give nothing more).  Reading used: in a hash layer the k
 * experts of a token are not chosen by the logits but looked up from a fixed
 * table by the token's id, table[id][0..k-1] (k distinct experts, in slot
 * order); the weights are still the router's softmax probabilities,
 * renormalised over those k experts: w[j] = p[table[id][j]] / sum_j p[...].
 * logits and p are as in route_token.  Returns 0, or -1 if id is outside
 * [0, n_vocab).
 */
static int route_token_hashed(const double *xt, int n_embd, const float *router, const float *bias,
                              int n_expert, int top_k, const int32_t *table, int64_t n_vocab, int32_t id,
                              float *logits, double *p, int32_t *idx, double *w)
{
    if (id < 0 || id >= n_vocab)
        return -1;
    for (int e = 0; e < n_expert; ++e) {
        double s = 0.0;
        const float *r = router + (int64_t)e * n_embd;
        for (int i = 0; i < n_embd; ++i)
            s += xt[i] * (double)r[i];
        if (bias)
            s += (double)bias[e];
        logits[e] = (float)s;
    }
    double mx = -INFINITY;
    for (int e = 0; e < n_expert; ++e)
        if ((double)logits[e] > mx)
            mx = logits[e];
    double z = 0.0;
    for (int e = 0; e < n_expert; ++e) {
        p[e] = exp((double)logits[e] - mx);
        z += p[e];
    }
    for (int e = 0; e < n_expert; ++e)
        p[e] /= z;
    double sum = 0.0;
    for (int j = 0; j < top_k; ++j) {
        idx[j] = table[(int64_t)id * top_k + j];
        sum += p[idx[j]];
    }
    for (int j = 0; j < top_k; ++j)
        w[j] = p[idx[j]] / sum;
    return 0;
}

/*
 * Route n_tok tokens.  x: [n_tok][n_embd] bf16 bits (x_is_bf16) or fp32.
 * router: [n_expert][n_embd] fp32; bias: [n_expert] fp32 or NULL.
 * Outputs (any may be NULL): logits [n_tok][n_expert] fp32, idx [n_tok][top_k],
 * w [n_tok][top_k] fp32, w64 [n_tok][top_k] fp64.  Returns 0, or -1 on bad sizes.
 */
int oracle_route(const void *x, int x_is_bf16, int64_t n_tok, int n_embd, const float *router,
                 const float *bias, int n_expert, int top_k, float *logits, int32_t *idx, float *w,
                 double *w64)
{
    if (n_tok < 0 || n_embd <= 0 || n_expert <= 0 || top_k <= 0 || top_k > n_expert)
        return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = 0; t < n_tok; ++t) {
        double *xt = malloc(sizeof(double) * n_embd);
        double *p = malloc(sizeof(double) * n_expert);
        float *lg = malloc(sizeof(float) * n_expert);
        int32_t *id = malloc(sizeof(int32_t) * top_k);
        double *wt = malloc(sizeof(double) * top_k);
        if (!xt || !p || !lg || !id || !wt) {
#pragma omp atomic write
            bad = 1;
        } else {
            for (int i = 0; i < n_embd; ++i)
                xt[i] = x_value(x, x_is_bf16, t * n_embd + i);
            route_token(xt, n_embd, router, bias, n_expert, top_k, lg, p, id, wt);
            for (int e = 0; e < n_expert; ++e)
                if (logits)
                    logits[t * n_expert + e] = lg[e];
            for (int j = 0; j < top_k; ++j) {
                if (idx)
                    idx[t * top_k + j] = id[j];
                if (w)
                    w[t * top_k + j] = (float)wt[j];
                if (w64)
                    w64[t * top_k + j] = wt[j];
            }
        }
        free(xt);
        free(p);
        free(lg);
        free(id);
        free(wt);
    }
    return bad ? -2 : 0;
}

/*
 * Hash-routed tokens (route_token_hashed): as oracle_route, with token_ids
 * [n_tok] and table [n_vocab][top_k].  Returns 0, -1 on bad sizes, -3 if an
 * id is out of range.
 */
int oracle_route_hashed(const void *x, int x_is_bf16, int64_t n_tok, int n_embd, const float *router,
                        const float *bias, int n_expert, int top_k, const int32_t *token_ids,
                        const int32_t *table, int64_t n_vocab, float *logits, int32_t *idx, float *w,
                        double *w64)
{
    if (n_tok < 0 || n_embd <= 0 || n_expert <= 0 || top_k <= 0 || top_k > n_expert || n_vocab <= 0)
        return -1;
    int bad = 0;
    for (int64_t t = 0; t < n_tok; ++t) {
        double *xt = malloc(sizeof(double) * n_embd);
        double *p = malloc(sizeof(double) * n_expert);
        float *lg = malloc(sizeof(float) * n_expert);
        int32_t *id = malloc(sizeof(int32_t) * top_k);
        double *wt = malloc(sizeof(double) * top_k);
        if (!xt || !p || !lg || !id || !wt) {
            bad = -2;
        } else {
            for (int i = 0; i < n_embd; ++i)
                xt[i] = x_value(x, x_is_bf16, t * n_embd + i);
            if (route_token_hashed(xt, n_embd, router, bias, n_expert, top_k, table, n_vocab, token_ids[t], lg,
                                   p, id, wt))
                bad = -3;
            else
                for (int j = 0; j < top_k; ++j) {
                    if (logits)
                        for (int e = 0; e < n_expert; ++e)
                            logits[t * n_expert + e] = lg[e];
                    if (idx)
                        idx[t * top_k + j] = id[j];
                    if (w)
                        w[t * top_k + j] = (float)wt[j];
                    if (w64)
                        w64[t * top_k + j] = wt[j];
                }
        }
        free(xt);
        free(p);
        free(lg);
        free(id);
        free(wt);
    }
    return bad;
}

/*
 * Per-expert token lists ([P1] section 3.3: experts are scheduled from the
 * router's output).  offsets[e]..offsets[e+1] delimit expert e's tokens in
 * `tokens`, which are in ascending token order.  offsets has n_expert+1
 * entries; tokens has n_tok*top_k.
 */
void oracle_bucket(const int32_t *idx, int64_t n_tok, int top_k, int n_expert, int32_t *offsets,
                   int32_t *tokens)
{
    int32_t pos = 0;
    for (int e = 0; e < n_expert; ++e) {
        offsets[e] = pos;
        for (int64_t t = 0; t < n_tok; ++t)
            for (int j = 0; j < top_k; ++j)
                if (idx[t * top_k + j] == e)
                    tokens[pos++] = (int32_t)t;
    }
    offsets[n_expert] = pos;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * One expert's SwiGLU feed-forward on one token, fp64 ([P1] section 3.2,
 * "MoE FFN"): g = Wg x, u = Wu x, h = SiLU(g) * u, y = Wd h.
 * wg, wu: [n_ff][n_embd] fp32; wd: [n_embd][n_ff] fp32.  h: scratch [n_ff].
 */
static void ffn_f32(const float *wg, const float *wu, const float *wd, const double *xt, int n_embd,
                    int n_ff, double *h, double *y)
{
    for (int f = 0; f < n_ff; ++f) {
        double g = 0.0, u = 0.0;
        const float *rg = wg + (int64_t)f * n_embd, *ru = wu + (int64_t)f * n_embd;
        for (int i = 0; i < n_embd; ++i) {
            g += (double)rg[i] * xt[i];
            u += (double)ru[i] * xt[i];
        }
        h[f] = silu(g) * u;
    }
    for (int r = 0; r < n_embd; ++r) {
        double s = 0.0;
        const float *rd = wd + (int64_t)r * n_ff;
        for (int f = 0; f < n_ff; ++f)
            s += (double)rd[f] * h[f];
        y[r] = s;
    }
}

/* Same with bf16 weights (the shared expert). */
static void ffn_bf16(const uint16_t *wg, const uint16_t *wu, const uint16_t *wd, const double *xt,
                     int n_embd, int n_ff, double *h, double *y)
{
    for (int f = 0; f < n_ff; ++f) {
        double g = 0.0, u = 0.0;
        const uint16_t *rg = wg + (int64_t)f * n_embd, *ru = wu + (int64_t)f * n_embd;
        for (int i = 0; i < n_embd; ++i) {
            g += bf16_value(rg[i]) * xt[i];
            u += bf16_value(ru[i]) * xt[i];
        }
        h[f] = silu(g) * u;
    }
    for (int r = 0; r < n_embd; ++r) {
        double s = 0.0;
        const uint16_t *rd = wd + (int64_t)r * n_ff;
        for (int f = 0; f < n_ff; ++f)
            s += bf16_value(rd[f]) * h[f];
        y[r] = s;
    }
}

/*
 * The block's output for the tokens listed in `rows` ([P1] section 3.2: route,
 * compute only the routed experts, compute the shared expert on every token,
 * merge the routed and shared outputs; [P5] section 2.1: 6 routed + 1 shared).
 *
 *   out[r] = sum_j w[t][j] * FFN_{idx[t][j]}(x_t) + FFN_shared(x_t),  t = rows[r]
 *
 * Routing is computed here (route_token), with fp64 weights.  Routed weights
 * are decoded with oracle_dequant_iq2 / oracle_dequant_q2k, one expert at a
 * time; the work is spread over experts with OpenMP and summed per token in
 * slot order, so the result does not depend on the thread count.
 *
 * expert_format 0: gate, up are [n_expert][n_ff][n_embd/256] IQ2 blocks and down is
 * [n_expert][n_embd][n_ff/256] Q2_K blocks; expert_format 1: all three are Q4_K
 * blocks in the same shapes.  sh_*: bf16 bits or NULL when there is no shared expert.
 * out: [n_rows][n_embd] fp64, overwritten.  Optional outputs (NULL to skip):
 * idx_out [n_rows][top_k], w_out [n_rows][top_k] fp64.
 * hash_table (NULL for a learned-routing layer): [n_vocab][top_k], with
 * token_ids [n_tok] (indexed by the row's token): the layer routes by
 * route_token_hashed.
 * Returns 0, -1 on bad sizes, -2 on allocation failure, -3 on a token id out of range.
 */
int oracle_forward(int n_embd, int n_ff, int n_expert, int top_k, int expert_format, const float *router,
                   const float *bias, const uint8_t *gate, const uint8_t *up, const uint8_t *down,
                   const uint16_t *codebook, const uint16_t *sh_gate, const uint16_t *sh_up,
                   const uint16_t *sh_down, const void *x, int x_is_bf16, const int32_t *rows,
                   int64_t n_rows, const int32_t *token_ids, const int32_t *hash_table, int64_t n_vocab,
                   double *out, int32_t *idx_out, double *w_out)
{
    if (n_embd % QK || n_ff % QK || n_embd <= 0 || n_ff <= 0 || top_k <= 0 || top_k > n_expert ||
        n_rows < 0 || (expert_format != 0 && expert_format != 1))
        return -1;
    const int gu_bytes = expert_format ? 144 : 66, dn_bytes = expert_format ? 144 : 84;
    const int64_t gate_blocks = (int64_t)n_ff * (n_embd / QK);
    const int64_t down_blocks = (int64_t)n_embd * (n_ff / QK);

    double *xs = malloc(sizeof(double) * (size_t)(n_rows ? n_rows : 1) * n_embd);
    int32_t *idx = malloc(sizeof(int32_t) * (size_t)(n_rows ? n_rows : 1) * top_k);
    double *w = malloc(sizeof(double) * (size_t)(n_rows ? n_rows : 1) * top_k);
    double *ys = calloc((size_t)(n_rows ? n_rows : 1) * top_k * n_embd, sizeof(double));
    if (!xs || !idx || !w || !ys) {
        free(xs), free(idx), free(w), free(ys);
        return -2;
    }
    for (int64_t r = 0; r < n_rows; ++r)
        for (int i = 0; i < n_embd; ++i)
            xs[r * n_embd + i] = x_value(x, x_is_bf16, (int64_t)rows[r] * n_embd + i);

    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        float *lg = malloc(sizeof(float) * n_expert);
        double *p = malloc(sizeof(double) * n_expert);
        if (!lg || !p) {
#pragma omp atomic write
            bad = 1;
        } else if (hash_table) {
            if (route_token_hashed(xs + r * n_embd, n_embd, router, bias, n_expert, top_k, hash_table, n_vocab,
                                   token_ids[rows[r]], lg, p, idx + r * top_k, w + r * top_k)) {
#pragma omp atomic write
                bad = 3;
            }
        } else {
            route_token(xs + r * n_embd, n_embd, router, bias, n_expert, top_k, lg, p, idx + r * top_k,
                        w + r * top_k);
        }
        free(lg);
        free(p);
    }

    /* Routed experts: decode each touched expert once, run all its (token, slot) pairs. */
#pragma omp parallel for schedule(dynamic, 1)
    for (int e = 0; e < n_expert; ++e) {
        int used = 0;
        for (int64_t q = 0; q < n_rows * top_k; ++q)
            used |= idx[q] == e;
        if (!used || bad)
            continue;
        float *wg = malloc(sizeof(float) * (size_t)n_ff * n_embd);
        float *wu = malloc(sizeof(float) * (size_t)n_ff * n_embd);
        float *wd = malloc(sizeof(float) * (size_t)n_embd * n_ff);
        double *h = malloc(sizeof(double) * n_ff);
        if (!wg || !wu || !wd || !h) {
#pragma omp atomic write
            bad = 1;
        } else {
            if (expert_format == 1) {
                oracle_dequant_q4k(gate + (int64_t)e * gate_blocks * gu_bytes, gate_blocks, wg);
                oracle_dequant_q4k(up + (int64_t)e * gate_blocks * gu_bytes, gate_blocks, wu);
                oracle_dequant_q4k(down + (int64_t)e * down_blocks * dn_bytes, down_blocks, wd);
            } else {
                oracle_dequant_iq2(gate + (int64_t)e * gate_blocks * gu_bytes, gate_blocks, codebook, wg);
                oracle_dequant_iq2(up + (int64_t)e * gate_blocks * gu_bytes, gate_blocks, codebook, wu);
                oracle_dequant_q2k(down + (int64_t)e * down_blocks * dn_bytes, down_blocks, wd);
            }
            for (int64_t q = 0; q < n_rows * top_k; ++q)
                if (idx[q] == e)
                    ffn_f32(wg, wu, wd, xs + (q / top_k) * n_embd, n_embd, n_ff, h, ys + q * n_embd);
        }
        free(wg);
        free(wu);
        free(wd);
        free(h);
    }

    /* Shared expert (weight 1) and the merge, per token. */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        double *h = malloc(sizeof(double) * n_ff);
        double *ysh = calloc(n_embd, sizeof(double));
        if (!h || !ysh) {
#pragma omp atomic write
            bad = 1;
        } else if (!bad) {
            if (sh_gate && sh_up && sh_down)
                ffn_bf16(sh_gate, sh_up, sh_down, xs + r * n_embd, n_embd, n_ff, h, ysh);
            for (int i = 0; i < n_embd; ++i) {
                double acc = 0.0;
                for (int j = 0; j < top_k; ++j)
                    acc += w[r * top_k + j] * ys[(r * top_k + j) * n_embd + i];
                out[r * n_embd + i] = acc + ysh[i];
            }
        }
        free(h);
        free(ysh);
    }
    if (idx_out)
        memcpy(idx_out, idx, sizeof(int32_t) * n_rows * top_k);
    if (w_out)
        memcpy(w_out, w, sizeof(double) * n_rows * top_k);
    free(xs);
    free(idx);
    free(w);
    free(ys);
    return bad == 3 ? -3 : bad ? -2 : 0;
}

/*
 * RMSNorm with unit gain between stacked layers: x = h / sqrt(mean(h^2) + eps),
 * in fp64, rounded to bf16 (nearest, ties to even).  h: [n_tok][n_embd] fp32.
 * x_bf16: [n_tok][n_embd] bf16 bits; x64 (optional): the fp64 values.
 */
void oracle_rmsnorm(const float *h, int64_t n_tok, int n_embd, double eps, uint16_t *x_bf16, double *x64)
{
    for (int64_t t = 0; t < n_tok; ++t) {
        double ss = 0.0;
        for (int i = 0; i < n_embd; ++i)
            ss += (double)h[t * n_embd + i] * (double)h[t * n_embd + i];
        double denom = sqrt(ss / n_embd + eps);
        for (int i = 0; i < n_embd; ++i) {
            double v = (double)h[t * n_embd + i] / denom;
            if (x64)
                x64[t * n_embd + i] = v;
            if (x_bf16)
                x_bf16[t * n_embd + i] = bf16_round(v);
        }
    }
}

/* Number of OpenMP threads the oracle's parallel loops use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the number of OpenMP threads for later calls (timing only: the results
 * do not depend on it). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
