// route.hip - router: fp64-accumulated logits, softmax -> top-k -> renormalise,
// and the per-expert token lists.
//
// The router scores every expert for each token and only the chosen experts are
// computed ("ds4 深度实战...", section 3.2 "MoE FFN"); it is kept at full
// precision (same page, section 2.1); 6 of 256 experts per token ("Redis 作者
// 出手！ds4...", section 2.1).  The gating is softmax over all logits, the k
// largest (lower expert index first among equal logits), renormalised over the
// selected experts.  Since the softmax is strictly increasing in the logit, the
// selection is taken on the fp32 logits, and the renormalised weights are
// exp(L_j - L_max) / sum_i exp(L_i - L_max) over the selected experts, in fp64.
#include "common.h"

namespace ds4 {

constexpr int RT_WAVES = 4;         // waves per router workgroup (one K quarter each)
constexpr int RT_TOK = 16;          // tokens per router workgroup beyond 64 tokens (fp32 activations; bf16 ones take the batched router)
constexpr int ROUTE_SMALL_MAX = 64; // fused top-k/bucketing (a tail workgroup per token tile) up to this n_tok

template <bool XBF16>
__device__ __forceinline__ void load_x4(const void *x, int64_t off, double v[4]) {
    if (XBF16) {
        uint2 r = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(x) + off);
        v[0] = bf16_to_f32((uint16_t)(r.x & 0xFFFF));
        v[1] = bf16_to_f32((uint16_t)(r.x >> 16));
        v[2] = bf16_to_f32((uint16_t)(r.y & 0xFFFF));
        v[3] = bf16_to_f32((uint16_t)(r.y >> 16));
    } else {
        float4 r = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(x) + off);
        v[0] = r.x, v[1] = r.y, v[2] = r.z, v[3] = r.w;
    }
}

// Order-preserving key: larger logit first, then smaller expert index.
__device__ __forceinline__ uint64_t topk_key(float L, int e) {
    uint32_t u = __float_as_uint(L);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)(0xFFFF - e);
}

// The logit a key was made from.
__device__ __forceinline__ float key_logit(uint64_t key) {
    const uint32_t u = (uint32_t)(key >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint64_t o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

// Small-batch hand-offs between workgroups use 64-bit words: 32 data bits
// under the call's 32-bit tag (never 0, the workspace's initial value),
// stored and polled at agent scope.  A word is seen whole or not at all, so a
// consumer that finds the tag has the value: no fences (which would write
// back and invalidate the L2) and nothing to reset.
__device__ __forceinline__ unsigned long long rt_poll(const unsigned long long *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void rt_put(unsigned long long *p, uint32_t tag, uint32_t v) {
    __hip_atomic_store(p, ((unsigned long long)tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until word p carries the call's tag (bounded: W.spin_limit polls);
// false, with the call's tag recorded in the host-visible status word, if the
// wait expired.
__device__ __forceinline__ bool rt_wait(const Work &W, const unsigned long long *p, uint32_t tag,
                                        unsigned long long &v) {
    const uint32_t want = tag ^ W.want_xor;
    for (int spins = 0; (uint32_t)(v >> 32) != want; ++spins) {
        if (spins > W.spin_limit) {
            report_wait_expired(W, tag);
            return false;
        }
        __builtin_amdgcn_s_sleep(2);
        v = rt_poll(p);
    }
    return true;
}

// Renormalised weight of selection `lane` (< k) among the k selected logits
// (every lane holds all of them; selection 0 is the largest): one exp per lane
// relative to the largest, the denominator by a sum over the lanes (all 64
// lanes call it; lanes >= k add 0 and get a value that is not used).  It was
// a loop of k exps in every lane, about 2 us of fp64 work in the router's tail.
__device__ __forceinline__ float topk_weight(const float (&sel_L)[MAX_TOPK], int k, int lane) {
    float myL = sel_L[0];
#pragma unroll
    for (int j = 1; j < MAX_TOPK; ++j)
        if (j == lane) myL = sel_L[j];
    const double ex = lane < k ? exp((double)myL - (double)sel_L[0]) : 0.0;
    return (float)(ex / wave_sum_dpp(ex));
}

// Top-k + renormalised weights for token t, by one wavefront, from the tagged
// logits of this call; the selection also goes to the tagged itag words.  An
// expired wait poisons the token's weights with NaN.
__device__ void topk_tagged(const Work &W, const unsigned long long *__restrict__ ltag, int t, int NE, int k,
                            uint32_t tag, int32_t *__restrict__ idx, float *__restrict__ w,
                            unsigned long long *__restrict__ itag) {
    const int lane = threadIdx.x & 63;
    const unsigned long long *row = ltag + (int64_t)t * MAX_EXPERT;
    unsigned long long v[4];
    // all four words in flight at once each round (a word that already
    // carries the tag reads the same again), until all carry it; bounded
    const uint32_t want = tag ^ W.want_xor;
    bool ok = true;
    for (int spins = 0;; ++spins) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = rt_poll(row + min(lane + 64 * i, NE - 1));
        bool have = true;
#pragma unroll
        for (int i = 0; i < 4; ++i) have &= (uint32_t)(v[i] >> 32) == want;
        if (__all(have)) break;
        if (spins > W.spin_limit) {
            if (lane == 0) report_wait_expired(W, tag);
            ok = have;
            break;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    // DPP maxima and ballots: no cross-lane round trip through LDS
    uint32_t key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) key[i] = lane + 64 * i < NE ? logit_key32(__uint_as_float((uint32_t)v[i])) : 0u;
    const bool bad = __ballot(!ok) != 0ull;
    float sel_L[MAX_TOPK] = {};
    int sel_e[MAX_TOPK] = {};
    for (int j = 0; j < k; ++j) {
        uint32_t m;
        topk_round(key, m, sel_e[j]);
        sel_L[j] = key32_logit(m);
    }
    const float wj = topk_weight(sel_L, k, lane);
    int e = sel_e[0];
#pragma unroll
    for (int j = 1; j < MAX_TOPK; ++j)
        if (j == lane) e = sel_e[j];
    if (lane < k) {
        idx[(int64_t)t * k + lane] = e;
        w[(int64_t)t * k + lane] = bad ? __builtin_nanf("") : wj;
        rt_put(itag + (int64_t)t * MAX_TOPK + lane, tag, (uint32_t)e);
    }
}

// Top-k + renormalised weights for token t, by one wavefront.
__device__ void topk_token(const float *__restrict__ logits, int t, int NE, int k, int32_t *__restrict__ idx,
                           float *__restrict__ w) {
    const int lane = threadIdx.x & 63;
    uint32_t key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        key[i] = e < NE ? logit_key32(logits[(int64_t)t * NE + e]) : 0u;
    }
    float sel_L[MAX_TOPK] = {};
    int sel_e[MAX_TOPK] = {};
    for (int j = 0; j < k; ++j) {
        uint32_t m;
        topk_round(key, m, sel_e[j]);
        sel_L[j] = key32_logit(m);  // no reload: the key holds the logit
    }
    const float wj = topk_weight(sel_L, k, lane);
    int e = sel_e[0];
#pragma unroll
    for (int j = 1; j < MAX_TOPK; ++j)
        if (j == lane) e = sel_e[j];
    if (lane < k) {
        idx[(int64_t)t * k + lane] = e;
        w[(int64_t)t * k + lane] = wj;
    }
}

// Per-expert lists for small n_tok by one workgroup of 256 threads: counts,
// offsets, active experts, and the list entries t*k+j in ascending t within
// each expert.  The tagged selections are read into LDS once; every scan
// after that is over LDS.
constexpr int BS_MAXQ = ROUTE_SMALL_MAX * MAX_TOPK;
__device__ void bucket_small(const unsigned long long *__restrict__ itag, uint32_t tag, int n_tok, int k, int NE,
                             const Work &W) {
    __shared__ int sidx[BS_MAXQ];
    __shared__ int cnt[MAX_EXPERT];
    __shared__ int wtot[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nq = n_tok * k;
    for (int q = tid; q < nq; q += 256) {
        const unsigned long long *p = itag + (int64_t)(q / k) * MAX_TOPK + q % k;
        unsigned long long v = rt_poll(p);
        sidx[q] = rt_wait(W, p, tag, v) ? (int)(uint32_t)v : 0;  // an expired wait already poisoned the weights
    }
    cnt[tid] = 0;
    __syncthreads();
    for (int q = tid; q < nq; q += 256) atomicAdd(&cnt[sidx[q]], 1);
    __syncthreads();
    // exclusive scan over the experts (thread e holds expert e) and the
    // compaction of the active ones, by wave scans
    const int c = tid < NE ? cnt[tid] : 0;
    int v = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    const uint64_t am = __ballot(c > 0);
    if (lane == 63) wtot[wave] = v;
    __shared__ int wact[4];
    if (lane == 0) wact[wave] = __popcll(am);
    __syncthreads();
    int pre = 0, apre = 0;
    for (int w = 0; w < wave; ++w) pre += wtot[w], apre += wact[w];
    const int start = pre + v - c;
    if (tid < NE) {
        W.offsets[tid] = start;
        if (c > 0) W.active[1 + apre + __popcll(am & ((1ull << lane) - 1ull))] = tid;
    }
    if (tid == 255) {
        W.offsets[NE] = pre + v;
        W.active[0] = apre + __popcll(am);
    }
    // list entries, ascending within each expert: selection q = tid + 256 j
    // (group g = 4 j + wave of 64 consecutive selections) goes to its
    // expert's start plus the earlier selections of that expert: those of its
    // own group by a wave match, those of earlier groups from each group's
    // per-expert counts (written by the group's first lane of each expert).
    // A serial scan of all selections per expert took 5-10 us here.
    constexpr int BS_GROUPS = BS_MAXQ / 64;
    static_assert(BS_MAXQ <= 2 * 256 && MAX_EXPERT == 256, "two rounds of 256 selections, experts 8 bits");
    __shared__ int ghist[BS_GROUPS][MAX_EXPERT];
    __shared__ int estart[MAX_EXPERT];
    const int ng = (nq + 63) / 64;
    for (int i = tid; i < ng * MAX_EXPERT; i += 256) ghist[i / MAX_EXPERT][i % MAX_EXPERT] = 0;
    estart[tid] = start;
    __syncthreads();
    int rank[2] = {0, 0};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (256 * j >= nq) break;  // uniform
        const int q = tid + 256 * j;
        const bool in = q < nq;
        const int e = in ? sidx[q] : 0;
        const uint64_t m = wave_match_any((uint32_t)e, 8) & __ballot(in);
        const uint64_t below = m & ((1ull << lane) - 1ull);
        if (in && below == 0) ghist[4 * j + wave][e] = __popcll(m);
        rank[j] = __popcll(below);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int q = tid + 256 * j;
        if (q >= nq) break;
        const int e = sidx[q], g = 4 * j + wave;
        int r = rank[j];
        for (int h = 0; h < g; ++h) r += ghist[h][e];
        W.list[estart[e] + r] = q;
    }
}

// Logits of one expert (blockIdx.x) for TT tokens per workgroup, fp64
// accumulation.  Wave w covers K quarter w; lane l holds 4 values at
// 4 l + 256 j of it (j < 4: n_embd <= 4096).  All of a wave's loads are in
// flight together (unconditional: tokens past the tile's end re-read its last
// token, chunks past the quarter re-read its first; neither is summed), and
// the quarters are added in order by wave 0.
// With fuse_tail, the grid has one more column: its workgroup in row y takes
// token tile y's top-k from the tagged logits, and (fuse_tail 1) the last of
// those tails builds the per-expert lists; with fuse_tail 2 the lists are
// left to the kernels that follow (the small-batch kernels build them from
// the selections).  A tail is dispatched after its tile's expert workgroups
// (row-major order) and waits only on them, so it never holds up their start.
constexpr int RT_KCH = 4;  // 256-value chunks per wave at most
template <bool XBF16, int TT>
__global__ __launch_bounds__(256) void k_route_logits(const float *__restrict__ R, const float *__restrict__ bias,
                                                      const void *__restrict__ x, int n_tok, int NE, int E,
                                                      int k, Work W, int fuse_tail, uint32_t tag) {
    __shared__ double part[RT_WAVES][TT];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.x;
    const int t0 = blockIdx.y * TT;
    const int nt = min(TT, n_tok - t0);
    if (fuse_tail && e == NE) {
        // the token tile's tail (the grid's extra column, dispatched after the
        // tile's expert workgroups): polls the tile's tagged logits from the
        // start, then takes each token's top-k.  No tickets: 256 workgroups
        // taking one from the same counter queued for microseconds
        for (int t = t0 + wave; t < t0 + nt; t += RT_WAVES) topk_tagged(W, W.ltag, t, NE, k, tag, W.idx, W.w, W.itag);
        if (fuse_tail == 2) return;
        // the lists: the last of the tails (a ticket among the gridDim.y of
        // them; the last taker resets it) polls every token's selection
        __shared__ int last;
        __syncthreads();
        if (threadIdx.x == 0) last = atomicAdd(&W.counters[0], 1) == (int)gridDim.y - 1;
        __syncthreads();
        if (!last) return;
        bucket_small(W.itag, tag, n_tok, k, NE, W);
        if (threadIdx.x == 0) W.counters[0] = 0;
        return;
    }
    const int kq = E / RT_WAVES, kb = wave * kq;
    {
        double acc[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[t] = 0.0;
        float4 r[RT_KCH];
        double xv[RT_KCH][TT][4];
#pragma unroll
        for (int j = 0; j < RT_KCH; ++j) {
            const int off = 4 * lane + 256 * j;
            const int i = kb + (off < kq ? off : 0);
            r[j] = *reinterpret_cast<const float4 *>(R + (int64_t)e * E + i);
#pragma unroll
            for (int t = 0; t < TT; ++t) load_x4<XBF16>(x, (int64_t)(t0 + min(t, nt - 1)) * E + i, xv[j][t]);
        }
#pragma unroll
        for (int j = 0; j < RT_KCH; ++j) {
            if (4 * lane + 256 * j < kq) {
#pragma unroll
                for (int t = 0; t < TT; ++t) {
                    acc[t] = fma(xv[j][t][0], (double)r[j].x, acc[t]);
                    acc[t] = fma(xv[j][t][1], (double)r[j].y, acc[t]);
                    acc[t] = fma(xv[j][t][2], (double)r[j].z, acc[t]);
                    acc[t] = fma(xv[j][t][3], (double)r[j].w, acc[t]);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const double s = wave_sum_dpp(acc[t]);
            if (lane == 0) part[wave][t] = s;
        }
    }
    __syncthreads();
    if (wave == 0 && lane < nt) {
        const double b = bias ? (double)bias[e] : 0.0;
        double s = part[0][lane];
#pragma unroll
        for (int w = 1; w < RT_WAVES; ++w) s += part[w][lane];
        const float L = (float)(s + b);
        if (fuse_tail)
            rt_put(W.ltag + (int64_t)(t0 + lane) * MAX_EXPERT + e, tag, __float_as_uint(L));
        else
            W.logits[(int64_t)(t0 + lane) * NE + e] = L;
    }
}

// Top-k for many tokens: one wavefront per token.
__global__ __launch_bounds__(256) void k_topk(int n_tok, int NE, int k, Work W) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t < n_tok) topk_token(W.logits, t, NE, k, W.idx, W.w);
}

// Per-expert token lists for any n_tok, by one workgroup of 1024 threads:
// a histogram and a scan give the offsets and the active experts; each chunk
// of 2048 tokens is marked in a per-expert bitmap (with the chunk's expert
// indices staged in LDS), and each expert's set bits are emitted in ascending
// token order as list entries t*k + j.
constexpr int BK_CHUNK = 2048;
constexpr int BK_WORDS = BK_CHUNK / 32;

// Exclusive prefix sum over the first 256 threads (4 waves) of the workgroup;
// every thread of the workgroup gets the total.  Uses wtot[4] of LDS.
__device__ __forceinline__ int scan256(int v, int tid, int *wtot, int &total) {
    const int lane = tid & 63, wave = tid >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (tid < 256 && lane == 63) wtot[wave] = x;
    __syncthreads();
    int pre = 0;
    for (int w = 0; w < wave && w < 4; ++w) pre += wtot[w];
    total = wtot[0] + wtot[1] + wtot[2] + wtot[3];
    __syncthreads();
    return pre + x - v;
}

__global__ __launch_bounds__(1024) void k_bucket(int n_tok, int NE, int k, Work W) {
    __shared__ uint32_t bitmap[MAX_EXPERT * BK_WORDS];  // 64 KB
    __shared__ uint8_t eidx[BK_CHUNK * MAX_TOPK];       // 16 KB: expert of every slot of the chunk
    __shared__ int cnt[MAX_EXPERT];
    __shared__ int base[MAX_EXPERT];
    __shared__ int part[MAX_EXPERT * 4];
    __shared__ int wtot[4];
    const int tid = threadIdx.x;
    const int nq = n_tok * k;
    for (int e = tid; e < MAX_EXPERT; e += 1024) cnt[e] = 0;
    __syncthreads();
    for (int q = tid; q < nq; q += 1024) atomicAdd(&cnt[W.idx[q]], 1);
    __syncthreads();
    {
        const int c = (tid < NE) ? cnt[tid] : 0;
        int total, nact;
        const int off = scan256(c, tid, wtot, total);
        const int apos = scan256(c > 0 ? 1 : 0, tid, wtot, nact);
        if (tid < NE) {
            base[tid] = off;
            W.offsets[tid] = off;
            if (c > 0) W.active[1 + apos] = tid;
        }
        if (tid == 0) {
            W.offsets[NE] = total;
            W.active[0] = nact;
        }
    }
    __syncthreads();
    for (int c0 = 0; c0 < n_tok; c0 += BK_CHUNK) {
        const int c1 = min(n_tok, c0 + BK_CHUNK);
        for (int i = tid; i < NE * BK_WORDS; i += 1024) bitmap[i] = 0u;
        __syncthreads();
        for (int q = c0 * k + tid; q < c1 * k; q += 1024) {
            const int e = W.idx[q];
            const int t = q / k - c0;
            eidx[q - c0 * k] = (uint8_t)e;
            atomicOr(&bitmap[e * BK_WORDS + (t >> 5)], 1u << (t & 31));
        }
        __syncthreads();
        // 4 threads per expert row, 16 words each
        const int e = tid >> 2, pr = tid & 3;
        int mine = 0;
        if (e < NE)
            for (int wd = 0; wd < BK_WORDS / 4; ++wd) mine += __popc(bitmap[e * BK_WORDS + pr * (BK_WORDS / 4) + wd]);
        part[tid] = mine;
        __syncthreads();
        if (e < NE) {
            int pos = base[e];
            for (int p = 0; p < pr; ++p) pos += part[e * 4 + p];
            for (int wd = 0; wd < BK_WORDS / 4; ++wd) {
                const int word = pr * (BK_WORDS / 4) + wd;
                uint32_t bits = bitmap[e * BK_WORDS + word];
                while (bits) {
                    const int b = __ffs(bits) - 1;
                    bits &= bits - 1;
                    const int tl = word * 32 + b;
                    int j = 0;
                    for (int jj = 0; jj < k; ++jj)
                        if (eidx[tl * k + jj] == (uint8_t)e) j = jj;
                    W.list[pos++] = (c0 + tl) * k + j;
                }
            }
        }
        __syncthreads();
        if (e < NE && pr == 0) base[e] += part[e * 4] + part[e * 4 + 1] + part[e * 4 + 2] + part[e * 4 + 3];
        __syncthreads();
    }
}

// ---------------------------------------------------------------- batched router
// For many tokens the router runs as an estimate plus an exact recomputation:
//  1. estimate: the fp32 router is split once into bf16 parts hi + mid + lo
//     and the logits are accumulated by bf16 MFMAs (products exact, fp32 sums
//     over 256-K chunks, chunk sums in fp64).  Each MFMA adds at most 32
//     roundings of at most 2^-23 relative to its running magnitude, 24 MFMAs
//     per chunk, so |estimate - exact| <= 800 * 2^-23 * sum_i |x_i| |w_i| (1 + 2^-7)
//     <= RT_BOUND * ||x|| * ||w_e|| (Cauchy-Schwarz), plus an absolute 1e-30
//     for flushed subnormal products.
//  2. per token, the k-th largest lower bound theta; every expert of the exact
//     top-k has an upper bound >= theta minus a few fp32 ulps (fp32 rounding
//     is monotone, and experts whose exact logits differ by more than an ulp
//     keep their order), so only experts above that are candidates.
//  3. the candidates' logits are recomputed in fp64 and rounded to fp32 exactly
//     as the single-token path does, and the top-k and the renormalised
//     weights are taken among them.
constexpr double RT_BOUND = 1.0e-4;

// One workgroup per expert: bf16 parts and the row norm (rounded up).
__global__ __launch_bounds__(256) void k_router_prep(const float *__restrict__ R, int NE, int E,
                                                     uint16_t *__restrict__ hml, float *__restrict__ norm) {
    __shared__ double red[4];
    const int e = blockIdx.x, tid = threadIdx.x;
    double ss = 0.0;
    for (int i = tid; i < E; i += 256) {
        const float w = R[(int64_t)e * E + i];
        const uint16_t hi = f32_to_bf16_rne(w);
        const float r1 = w - bf16_to_f32(hi);
        const uint16_t mid = f32_to_bf16_rne(r1);
        const float r2 = r1 - bf16_to_f32(mid);
        const uint16_t lo = f32_to_bf16_rne(r2);
        hml[((int64_t)0 * NE + e) * E + i] = hi;
        hml[((int64_t)1 * NE + e) * E + i] = mid;
        hml[((int64_t)2 * NE + e) * E + i] = lo;
        ss = fma((double)w, (double)w, ss);
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    if (tid == 0) norm[e] = (float)(sqrt(red[0] + red[1] + red[2] + red[3]) * (1.0 + 1e-6));
}

hipError_t launch_router_prep(const float *router, int NE, int E, uint16_t *hml, float *norm, hipStream_t s) {
    hipLaunchKernelGGL(k_router_prep, dim3(NE), dim3(256), 0, s, router, NE, E, hml, norm);
    return hipGetLastError();
}

typedef __bf16 rt_bf16x8 __attribute__((ext_vector_type(8)));
typedef float rt_floatx4 __attribute__((ext_vector_type(4)));

// Estimates, split over K: workgroup (expert tile, token tile, K quarter)
// covers 64 experts x 64 tokens x n_embd / 4; wave w takes experts
// 16 w..16 w+15 (B: lane l holds expert l % 16, K 8 (l / 16)..+8, for each of
// the three router parts) and the four 16-token tiles (A: token l % 16 of the
// tile, the same K).  The quarter sums go to est[quarter][token][expert] and
// are added in fp64 by the selection.  The first workgroup also clears the
// per-expert counters that the selection fills.
constexpr int RA_SPLIT = 4;
__global__ __launch_bounds__(256) void k_route_approx(const uint16_t *__restrict__ hml, const uint16_t *__restrict__ x,
                                                      int n_tok, int NE, int E, float *__restrict__ est,
                                                      int32_t *__restrict__ ecount) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rl = lane & 15, grp = lane >> 4;
    if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
        for (int i = threadIdx.x; i < NE; i += 256) ecount[i] = 0;
    const int e = blockIdx.x * 64 + wave * 16 + rl;
    const int t0 = blockIdx.y * 64;
    const bool eok = e < NE;
    const int kq = E / RA_SPLIT, kb = blockIdx.z * kq;
    const uint16_t *wp[3];
#pragma unroll
    for (int p = 0; p < 3; ++p) wp[p] = hml + ((int64_t)p * NE + (eok ? e : 0)) * E + kb + 8 * grp;
    // every load is unconditional: tokens past n_tok read token 0 and experts
    // past NE read expert 0 (in bounds); their products land in accumulator
    // rows and columns that are never stored.
    // x (64 tokens x 64 K per stage) is staged in LDS once for the four waves,
    // double-buffered with one barrier per stage: thread t moves 32 bytes of
    // row t / 4, 16-byte units 2 (t % 4) and 2 (t % 4) + 1.  Unit u of row r
    // sits at position u ^ (r & 7), so a step's A reads hit distinct banks.
    __shared__ uint4 xs[2][64 * 8];
    const int sr = threadIdx.x >> 2, su = 2 * (threadIdx.x & 3);
    const uint16_t *xsrc = x + (int64_t)(t0 + sr < n_tok ? t0 + sr : 0) * E + kb + 8 * su;
    double acc[4][4] = {};
    // router parts: 32-K steps, two per stage, one stage ahead in named
    // buffers that alternate (no copies).  The fp32 MFMA sums go into the fp64
    // accumulators every 256 K.
    struct Stage {
        uint4 b[2][3];
    };
    const int nst = kq / 64;  // a multiple of 4: the launch requires n_embd % 1024 == 0
    auto loadb = [&](int st, Stage &g) __attribute__((always_inline)) {
        const int s0 = min(st, nst - 1) * 64;  // past the end: the last stage again, unused
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int p = 0; p < 3; ++p) g.b[s][p] = *reinterpret_cast<const uint4 *>(wp[p] + s0 + 32 * s);
    };
    uint4 xr0, xr1;  // x of the next stage, on its way to LDS
    auto loadx = [&](int st) __attribute__((always_inline)) {
        const int s0 = min(st, nst - 1) * 64;
        xr0 = *reinterpret_cast<const uint4 *>(xsrc + s0);
        xr1 = *reinterpret_cast<const uint4 *>(xsrc + s0 + 8);
    };
    auto storex = [&](int buf) __attribute__((always_inline)) {
        xs[buf][sr * 8 + (su ^ (sr & 7))] = xr0;
        xs[buf][sr * 8 + ((su + 1) ^ (sr & 7))] = xr1;
    };
    rt_floatx4 part[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) part[i] = rt_floatx4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int st, const Stage &g) __attribute__((always_inline)) {
        const uint4 *xb = xs[st & 1];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 a = xb[(16 * i + rl) * 8 + ((4 * s + grp) ^ (rl & 7))];
#pragma unroll
                for (int p = 0; p < 3; ++p)
                    part[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(rt_bf16x8, a),
                                                                      __builtin_bit_cast(rt_bf16x8, g.b[s][p]),
                                                                      part[i], 0, 0, 0);
            }
        if ((st & 3) == 3) {  // 256 K done
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[i][v] += (double)part[i][v];
                part[i] = rt_floatx4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    // one stage: compute st; put x of st + 1 (loaded a stage ago) into the
    // other buffer, whose readers finished before the last barrier; load x
    // and the router parts of st + 2
    auto stage = [&](int st, Stage &g) __attribute__((always_inline)) {
        compute(st, g);
        if (st + 1 < nst) storex((st + 1) & 1);
        loadx(st + 2);
        loadb(st + 2, g);
        __syncthreads();
    };
    Stage g0, g1;
    loadx(0);
    loadb(0, g0);
    storex(0);
    loadx(1);
    loadb(1, g1);
    __syncthreads();
    for (int st = 0; st < nst; st += 2) {
        stage(st, g0);
        stage(st + 1, g1);
    }
    // C layout: lane (rl, grp) holds tokens 4 grp + v of each tile for expert rl
    float *eq = est + (int64_t)blockIdx.z * n_tok * NE;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int t = t0 + 16 * i + 4 * grp + v;
            if (t < n_tok && eok) eq[(int64_t)t * NE + e] = (float)acc[i][v];
        }
}

// One wavefront per token: bounds, candidates, exact fp64 logits of the
// candidates, top-k and renormalised weights.  Lane l holds x at 4 l + 256 m.
constexpr int RS_MAXV = 4096 / 64;   // x values per lane (n_embd <= 4096)
__global__ __launch_bounds__(256) void k_route_select(const float *__restrict__ R, const float *__restrict__ bias,
                                                      const float *__restrict__ rnorm, const uint16_t *__restrict__ x,
                                                      int n_tok, int NE, int E, int k, Work W) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= n_tok) return;
    const int nm = E / 256;
    float xv[RS_MAXV];
    double ss = 0.0;
    // loads are unconditional (chunks past n_embd re-read the last one and
    // are zeroed), so they are all in flight at once
    uint2 xr[RS_MAXV / 4];
#pragma unroll
    for (int m = 0; m < RS_MAXV / 4; ++m)
        xr[m] = *reinterpret_cast<const uint2 *>(x + (int64_t)t * E + 256 * min(m, nm - 1) + 4 * lane);
#pragma unroll
    for (int m = 0; m < RS_MAXV / 4; ++m) {
        const bool in = m < nm;
        xv[4 * m + 0] = in ? bf16_to_f32((uint16_t)(xr[m].x & 0xFFFF)) : 0.0f;
        xv[4 * m + 1] = in ? bf16_to_f32((uint16_t)(xr[m].x >> 16)) : 0.0f;
        xv[4 * m + 2] = in ? bf16_to_f32((uint16_t)(xr[m].y & 0xFFFF)) : 0.0f;
        xv[4 * m + 3] = in ? bf16_to_f32((uint16_t)(xr[m].y >> 16)) : 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) ss = fma((double)xv[4 * m + j], (double)xv[4 * m + j], ss);
    }
    const double xn = sqrt(wave_sum_dpp(ss)) * (1.0 + 1e-12);
    // bounds of every expert (lane l: experts l + 64 i)
    double lb[4], ub[4], bb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        if (e < NE) {
            bb[i] = bias ? (double)bias[e] : 0.0;
            double a = bb[i];
#pragma unroll
            for (int qd = 0; qd < RA_SPLIT; ++qd) a += (double)W.rest[((int64_t)qd * n_tok + t) * NE + e];
            const double del = RT_BOUND * xn * (double)rnorm[e] + 1e-30;
            lb[i] = a - del;
            ub[i] = a + del;
        } else {
            bb[i] = 0.0, lb[i] = -INFINITY, ub[i] = -INFINITY;
        }
    }
    // theta = k-th largest lower bound
    double theta = -INFINITY;
    {
        bool taken[4] = {false, false, false, false};
        for (int j = 0; j < k; ++j) {
            double best = -INFINITY;
            int bi = -1;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (!taken[i] && lb[i] > best) best = lb[i], bi = i;
            const double m = wave_max_dpp(best);
            theta = m;
            // the lowest lane holding the maximum gives it up
            const uint64_t holders = __ballot(bi >= 0 && best == m);
            const int who = __ffsll((unsigned long long)holders) - 1;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (lane == who && bi == i) taken[i] = true;
        }
    }
    const double cut = theta - (fabs(theta) * 0x1p-20 + 1e-30);
    // candidates (upper bound at or above the cut), in ascending expert order,
    // into this wave's LDS list (a wave's LDS accesses complete in order)
    __shared__ int clist[4][MAX_EXPERT];
    int *cl = clist[threadIdx.x >> 6];
    int ncand = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool in = ub[i] >= cut;
        const uint64_t cm = __ballot(in);
        if (in) cl[ncand + __popcll(cm & ((1ull << lane) - 1ull))] = lane + 64 * i;
        ncand += __popcll(cm);
    }
    // exact logits of the candidates, one row at a time: its 16-byte chunks
    // are all in flight at once (chunks past n_embd re-read the last one,
    // where xv is zero)
    uint64_t key[4];
    float Lv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) key[i] = 0ull, Lv[i] = 0.f;
    for (int c = 0; c < ncand; ++c) {
        const int e = cl[c];
        const float *rp = R + (int64_t)e * E + 4 * lane;
        float4 r[RS_MAXV / 4];
#pragma unroll
        for (int m = 0; m < RS_MAXV / 4; ++m) r[m] = *reinterpret_cast<const float4 *>(rp + 256 * min(m, nm - 1));
        double s0 = 0.0, s1 = 0.0;
#pragma unroll
        for (int m = 0; m < RS_MAXV / 4; m += 2) {
            s0 = fma((double)xv[4 * m + 0], (double)r[m].x, s0);
            s0 = fma((double)xv[4 * m + 1], (double)r[m].y, s0);
            s0 = fma((double)xv[4 * m + 2], (double)r[m].z, s0);
            s0 = fma((double)xv[4 * m + 3], (double)r[m].w, s0);
            s1 = fma((double)xv[4 * m + 4], (double)r[m + 1].x, s1);
            s1 = fma((double)xv[4 * m + 5], (double)r[m + 1].y, s1);
            s1 = fma((double)xv[4 * m + 6], (double)r[m + 1].z, s1);
            s1 = fma((double)xv[4 * m + 7], (double)r[m + 1].w, s1);
        }
        const double sv = wave_sum_dpp(s0 + s1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (lane + 64 * i == e) {
                Lv[i] = (float)(sv + bb[i]);
                key[i] = topk_key(Lv[i], e);
            }
    }
    // top-k among the candidates, renormalised weights
    float sel_L[MAX_TOPK] = {};
    int sel_e[MAX_TOPK] = {};
    for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < 4; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
        const int e = 0xFFFF - (int)(best & 0xFFFFu);
        sel_e[j] = e;
        float Le = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (lane + 64 * i == e) Le = Lv[i], key[i] = 0ull;
        sel_L[j] = __shfl(Le, e & 63, 64);
    }
    const float wj = topk_weight(sel_L, k, lane);
    int e = sel_e[0];
#pragma unroll
    for (int j = 1; j < MAX_TOPK; ++j)
        if (j == lane) e = sel_e[j];
    if (lane < k) {
        W.idx[(int64_t)t * k + lane] = e;
        W.w[(int64_t)t * k + lane] = wj;
        atomicAdd(&W.ecount[e], 1);
    }
}

// Per-expert lists after the batched selection: one workgroup per expert.
// The expert's offset and its rank among the active experts come from the
// counts of the lower experts; its entries t*k + j are emitted in ascending t
// by a workgroup-wide scan over the tokens.
__global__ __launch_bounds__(256) void k_fill_lists(int n_tok, int NE, int k, Work W) {
    __shared__ int wtot[4];
    const int e = blockIdx.x, tid = threadIdx.x;
    int total, off, nact, apos;
    {
        const int c = (tid < NE) ? W.ecount[tid] : 0;
        const int ex = scan256(c, tid, wtot, total);
        const int ax = scan256(c > 0 ? 1 : 0, tid, wtot, nact);
        __shared__ int mine[2];
        if (tid == e) mine[0] = ex, mine[1] = ax;
        __syncthreads();
        off = mine[0], apos = mine[1];
    }
    const int cnt = W.ecount[e];
    if (tid == 0) {
        W.offsets[e] = off;
        if (cnt > 0) W.active[1 + apos] = e;
        if (e == NE - 1) {
            W.offsets[NE] = total;
            W.active[0] = nact;
        }
    }
    if (cnt == 0) return;
    int run = off;
    for (int t0 = 0; t0 < n_tok; t0 += 256) {
        const int t = t0 + tid;
        int j = -1;
        if (t < n_tok)
            for (int jj = 0; jj < k; ++jj)
                if (W.idx[(int64_t)t * k + jj] == e) j = jj;
        int tot;
        const int pos = scan256(j >= 0 ? 1 : 0, tid, wtot, tot);
        if (j >= 0) W.list[run + pos] = t * k + j;
        run += tot;
    }
}

// ---------------------------------------------------------------- hash-routed layers
// A hash layer takes a token's experts from row `id` of its table, in slot
// order, and weights them by the softmax over all logits renormalised over
// those experts.  The renormalisation cancels every other expert:
// p_j / sum_i p_i = exp(L_j - M) / sum_i exp(L_i - M) over the k table experts
// alone (M: their largest logit), so only k router rows are read per token.
// One workgroup per token; wave w computes the logits of slots w, w + 4
// (fp64 accumulation, rounded to fp32 as in the learned router).  An id
// outside [0, n_vocab) poisons the token's weights with NaN (its experts are
// then row 0's, so every later access stays in bounds) and records the call
// in the host-visible status word.
template <bool XBF16>
__global__ __launch_bounds__(256) void k_route_hashed(const float *__restrict__ R, const float *__restrict__ bias,
                                                      const void *__restrict__ x, const int32_t *__restrict__ table,
                                                      int n_vocab, int E, int k, Work W, uint32_t tag) {
    __shared__ float Ls[MAX_TOPK];
    __shared__ int Es[MAX_TOPK];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x;
    const int id = W.ids[t];
    const bool bad = id < 0 || id >= n_vocab;
    const int32_t *row = table + (int64_t)(bad ? 0 : id) * k;
    for (int j = wave; j < k; j += RT_WAVES) {
        const int e = row[j];
        double acc = 0.0;
        for (int i = 4 * lane; i < E; i += 256) {
            const float4 r = *reinterpret_cast<const float4 *>(R + (int64_t)e * E + i);
            double xv[4];
            load_x4<XBF16>(x, (int64_t)t * E + i, xv);
            acc = fma(xv[0], (double)r.x, acc);
            acc = fma(xv[1], (double)r.y, acc);
            acc = fma(xv[2], (double)r.z, acc);
            acc = fma(xv[3], (double)r.w, acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) {
            Ls[j] = (float)(acc + (bias ? (double)bias[e] : 0.0));
            Es[j] = e;
        }
    }
    __syncthreads();
    if (wave == 0 && lane < k) {
        float m = Ls[0];
        for (int j = 1; j < k; ++j) m = fmaxf(m, Ls[j]);
        double z = 0.0, num = 0.0;
        for (int j = 0; j < k; ++j) {
            const double ex = exp((double)Ls[j] - (double)m);
            z += ex;
            if (j == lane) num = ex;
        }
        W.idx[(int64_t)t * k + lane] = Es[lane];
        W.w[(int64_t)t * k + lane] = bad ? __builtin_nanf("") : (float)(num / z);
    }
    if (bad && threadIdx.x == 0) report_bad_id(W, tag);
}

hipError_t launch_route(const Layer &L, const Work &W, const void *x, int n_tok, hipStream_t s,
                        unsigned long long ep, bool lists) {
    const uint32_t tag = (uint32_t)(ep % 0xFFFFFFFFull) + 1u;
    const int NE = L.n_expert;
    if (L.hash_table) {
        // table lookups and k logits per token, then the per-expert lists
        if (L.act_dtype == 1)
            hipLaunchKernelGGL(k_route_hashed<true>, dim3(n_tok), dim3(256), 0, s, L.router, L.router_bias, x,
                               L.hash_table, L.n_vocab, L.n_embd, L.top_k, W, tag);
        else
            hipLaunchKernelGGL(k_route_hashed<false>, dim3(n_tok), dim3(256), 0, s, L.router, L.router_bias, x,
                               L.hash_table, L.n_vocab, L.n_embd, L.top_k, W, tag);
        hipLaunchKernelGGL(k_bucket, dim3(1), dim3(1024), 0, s, n_tok, NE, L.top_k, W);
        return hipGetLastError();
    }
    if (n_tok > ROUTE_SMALL_MAX && L.act_dtype == 1 && L.n_embd % (4 * QK) == 0) {
        // batched: MFMA estimates, exact candidates, lists
        const uint16_t *xb = static_cast<const uint16_t *>(x);
        hipLaunchKernelGGL(k_route_approx, dim3((NE + 63) / 64, (n_tok + 63) / 64, RA_SPLIT), dim3(256), 0, s,
                           L.router_hml, xb, n_tok, NE, L.n_embd, W.rest, W.ecount);
        hipLaunchKernelGGL(k_route_select, dim3((n_tok + 3) / 4), dim3(256), 0, s, L.router, L.router_bias,
                           L.router_norm, xb, n_tok, NE, L.n_embd, L.top_k, W);
        hipLaunchKernelGGL(k_fill_lists, dim3(NE), dim3(256), 0, s, n_tok, NE, L.top_k, W);
        return hipGetLastError();
    }
    const int fuse = n_tok <= ROUTE_SMALL_MAX ? (lists ? 1 : 2) : 0;
    // token tiles of 1, 2 or 4 for calls of up to 8 tokens (a larger tile
    // would load and multiply clamped copies of the last token; 4-token tiles
    // at 5..8 tokens let two tiles' tail workgroups take the top-k side by
    // side), and 8 up to 64 tokens: the 16-token tile takes 252 VGPRs (2 waves
    // per SIMD), and 8-token tiles measured 44 -> 33 us at 16 tokens, 52 -> 47
    // at 32
    const int tt = n_tok == 1 ? 1 : n_tok == 2 ? 2 : n_tok <= 8 ? 4 : fuse ? 8 : RT_TOK;
    // with the fused tail, one more workgroup per token tile takes its top-k
    const dim3 grid(NE + (fuse ? 1 : 0), (n_tok + tt - 1) / tt);
    const bool bf = L.act_dtype == 1;
#define DS4_ROUTE_LAUNCH(T)                                                                                   \
    hipLaunchKernelGGL((bf ? k_route_logits<true, T> : k_route_logits<false, T>), grid, dim3(256), 0, s, L.router, \
                       L.router_bias, x, n_tok, NE, L.n_embd, L.top_k, W, fuse, tag)
    switch (tt) {
        case 1: DS4_ROUTE_LAUNCH(1); break;
        case 2: DS4_ROUTE_LAUNCH(2); break;
        case 4: DS4_ROUTE_LAUNCH(4); break;
        case 8: DS4_ROUTE_LAUNCH(8); break;
        default: DS4_ROUTE_LAUNCH(RT_TOK); break;
    }
#undef DS4_ROUTE_LAUNCH
    if (!fuse) {
        hipLaunchKernelGGL(k_topk, dim3((n_tok + 3) / 4), dim3(256), 0, s, n_tok, NE, L.top_k, W);
        hipLaunchKernelGGL(k_bucket, dim3(1), dim3(1024), 0, s, n_tok, NE, L.top_k, W);
    }
    return hipGetLastError();
}

// Fill n 32-bit words with a value (counters that must start at zero).
__global__ __launch_bounds__(256) void k_fill_u32(uint32_t *__restrict__ p, int n, uint32_t v) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = v;
}

hipError_t launch_fill_u32(uint32_t *p, int n, uint32_t v, hipStream_t s) {
    hipLaunchKernelGGL(k_fill_u32, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

// Copy the internal routing results into the caller's buffers.
__global__ void k_route_export(int n_tok, int NE, int k, Work W, int32_t *__restrict__ idx, float *__restrict__ w,
                               int32_t *__restrict__ offsets, int32_t *__restrict__ tokens) {
    const int nq = n_tok * k;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nq; i += gridDim.x * blockDim.x) {
        if (idx) idx[i] = W.idx[i];
        if (w) w[i] = W.w[i];
        if (tokens) tokens[i] = W.list[i] / k;
    }
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i <= NE; i += gridDim.x * blockDim.x)
        if (offsets) offsets[i] = W.offsets[i];
}

hipError_t launch_route_export(const Layer &L, const Work &W, int n_tok, int32_t *idx, float *w, int32_t *offsets,
                               int32_t *tokens, hipStream_t s) {
    int nq = n_tok * L.top_k;
    int grid = min(1024, (nq + 255) / 256 + 1);
    hipLaunchKernelGGL(k_route_export, dim3(grid), dim3(256), 0, s, n_tok, L.n_expert, L.top_k, W, idx, w,
                       offsets, tokens);
    return hipGetLastError();
}

}  // namespace ds4
