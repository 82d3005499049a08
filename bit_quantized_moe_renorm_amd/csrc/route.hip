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

constexpr int RT_WAVES = 4;         // experts per workgroup (one per wave)
constexpr int RT_TOK = 16;          // tokens per workgroup
constexpr int ROUTE_SMALL_MAX = 64; // fused top-k/bucketing in the last workgroup up to this n_tok

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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint64_t o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

// Top-k + renormalised weights for token t, by one wavefront.
__device__ void topk_token(const float *__restrict__ logits, int t, int NE, int k, int32_t *__restrict__ idx,
                           float *__restrict__ w) {
    const int lane = threadIdx.x & 63;
    uint64_t key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int e = lane + 64 * i;
        key[i] = (e < NE) ? topk_key(logits[(int64_t)t * NE + e], e) : 0ull;
    }
    float sel_L[MAX_TOPK];
    int sel_e[MAX_TOPK];
    for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < 4; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
        int e = 0xFFFF - (int)(best & 0xFFFFu);
        sel_e[j] = e;
        sel_L[j] = logits[(int64_t)t * NE + e];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (lane + 64 * i == e) key[i] = 0ull;
    }
    if (lane < k) {
        // every lane < k evaluates the common denominator; lane j also its numerator
        double m = (double)sel_L[0], z = 0.0, num = 0.0;
        for (int j = 0; j < k; ++j) {
            double ex = exp((double)sel_L[j] - m);
            z += ex;
            if (j == lane) num = ex;
        }
        int e = 0;
        for (int j = 0; j < k; ++j)
            if (j == lane) e = sel_e[j];
        idx[(int64_t)t * k + lane] = e;
        w[(int64_t)t * k + lane] = (float)(num / z);
    }
}

// Per-expert lists for small n_tok by one workgroup: counts, offsets, active
// experts, and the list entries t*k+j in ascending t within each expert.
__device__ void bucket_small(const int32_t *__restrict__ idx, int n_tok, int k, int NE, const Work &W) {
    __shared__ int cnt[MAX_EXPERT + 1];
    __shared__ int act[MAX_EXPERT + 1];
    const int tid = threadIdx.x;
    const int nq = n_tok * k;
    for (int e = tid; e < NE; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    for (int q = tid; q < nq; q += blockDim.x) atomicAdd(&cnt[idx[q]], 1);
    __syncthreads();
    if (tid == 0) {
        int run = 0, u = 0;
        for (int e = 0; e < NE; ++e) {
            int c = cnt[e];
            cnt[e] = run;
            W.offsets[e] = run;
            if (c) act[u++] = e;
            run += c;
        }
        W.offsets[NE] = run;
        W.active[0] = u;
        for (int i = 0; i < u; ++i) W.active[1 + i] = act[i];
    }
    __syncthreads();
    for (int e = tid; e < NE; e += blockDim.x) {
        int pos = cnt[e];
        for (int q = 0; q < nq; ++q)
            if (idx[q] == e) W.list[pos++] = q;
    }
}

// Logits for RT_WAVES experts x RT_TOK tokens per workgroup, fp64 accumulation.
// With fuse_tail, the last workgroup to finish also does top-k and bucketing.
template <bool XBF16>
__global__ __launch_bounds__(256) void k_route_logits(const float *__restrict__ R, const float *__restrict__ bias,
                                                      const void *__restrict__ x, int n_tok, int NE, int E,
                                                      int k, Work W, int fuse_tail) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.x * RT_WAVES + wave;
    const int t0 = blockIdx.y * RT_TOK;
    const int nt = min(RT_TOK, n_tok - t0);
    if (e < NE) {
        double acc[RT_TOK];
#pragma unroll
        for (int t = 0; t < RT_TOK; ++t) acc[t] = 0.0;
        for (int i = 4 * lane; i < E; i += 256) {
            float4 r = *reinterpret_cast<const float4 *>(R + (int64_t)e * E + i);
#pragma unroll
            for (int t = 0; t < RT_TOK; ++t) {
                if (t < nt) {
                    double xv[4];
                    load_x4<XBF16>(x, (int64_t)(t0 + t) * E + i, xv);
                    acc[t] = fma(xv[0], (double)r.x, acc[t]);
                    acc[t] = fma(xv[1], (double)r.y, acc[t]);
                    acc[t] = fma(xv[2], (double)r.z, acc[t]);
                    acc[t] = fma(xv[3], (double)r.w, acc[t]);
                }
            }
        }
        const double b = bias ? (double)bias[e] : 0.0;
#pragma unroll
        for (int t = 0; t < RT_TOK; ++t) {
            if (t < nt) {
                double s = wave_sum(acc[t]);
                if (lane == 0) W.logits[(int64_t)(t0 + t) * NE + e] = (float)(s + b);
            }
        }
    }
    if (!fuse_tail) return;
    // last-workgroup epilogue: release our logits, take a ticket
    __shared__ int last;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        int total = gridDim.x * gridDim.y;
        int ticket = atomicAdd(&W.counters[0], 1);
        last = (ticket == total - 1);
    }
    __syncthreads();
    if (!last) return;
    __threadfence();
    const int nw = blockDim.x >> 6;
    for (int t = wave; t < n_tok; t += nw) topk_token(W.logits, t, NE, k, W.idx, W.w);
    __threadfence();
    __syncthreads();
    bucket_small(W.idx, n_tok, k, NE, W);
    if (threadIdx.x == 0) W.counters[0] = 0;
}

// Top-k for many tokens: one wavefront per token.
__global__ __launch_bounds__(256) void k_topk(int n_tok, int NE, int k, Work W) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t < n_tok) topk_token(W.logits, t, NE, k, W.idx, W.w);
}

// Per-expert token lists for any n_tok, by one workgroup of 1024 threads:
// a histogram gives the offsets; each chunk of 2048 tokens is marked in a
// per-expert bitmap, and each expert's set bits are emitted in ascending order.
constexpr int BK_CHUNK = 2048;
constexpr int BK_WORDS = BK_CHUNK / 32;
__global__ __launch_bounds__(1024) void k_bucket(int n_tok, int NE, int k, Work W) {
    __shared__ uint32_t bitmap[MAX_EXPERT * BK_WORDS];  // 64 KB
    __shared__ int cnt[MAX_EXPERT + 1];
    __shared__ int base[MAX_EXPERT];
    __shared__ int part[MAX_EXPERT * 4];
    const int tid = threadIdx.x;
    const int nq = n_tok * k;
    for (int e = tid; e < NE; e += 1024) cnt[e] = 0;
    __syncthreads();
    for (int q = tid; q < nq; q += 1024) atomicAdd(&cnt[W.idx[q]], 1);
    __syncthreads();
    if (tid == 0) {
        int run = 0, u = 0;
        for (int e = 0; e < NE; ++e) {
            int c = cnt[e];
            base[e] = run;
            W.offsets[e] = run;
            if (c) W.active[1 + u++] = e;
            run += c;
        }
        W.offsets[NE] = run;
        W.active[0] = u;
    }
    __syncthreads();
    for (int c0 = 0; c0 < n_tok; c0 += BK_CHUNK) {
        const int c1 = min(n_tok, c0 + BK_CHUNK);
        for (int i = tid; i < NE * BK_WORDS; i += 1024) bitmap[i] = 0u;
        __syncthreads();
        for (int q = c0 * k + tid; q < c1 * k; q += 1024) {
            int t = q / k - c0;
            atomicOr(&bitmap[W.idx[q] * BK_WORDS + (t >> 5)], 1u << (t & 31));
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
                    int b = __ffs(bits) - 1;
                    bits &= bits - 1;
                    int t = c0 + word * 32 + b;
                    int j = 0;
                    for (int jj = 0; jj < k; ++jj)
                        if (W.idx[(int64_t)t * k + jj] == e) j = jj;
                    W.list[pos++] = t * k + j;
                }
            }
        }
        __syncthreads();
        if (e < NE && pr == 0) base[e] += part[e * 4] + part[e * 4 + 1] + part[e * 4 + 2] + part[e * 4 + 3];
        __syncthreads();
    }
}

hipError_t launch_route(const Layer &L, const Work &W, const void *x, int n_tok, hipStream_t s, hipEvent_t *ev) {
    const int NE = L.n_expert;
    dim3 grid((NE + RT_WAVES - 1) / RT_WAVES, (n_tok + RT_TOK - 1) / RT_TOK);
    const int fuse = n_tok <= ROUTE_SMALL_MAX;
    if (L.act_dtype == 1)
        hipLaunchKernelGGL(k_route_logits<true>, grid, dim3(256), 0, s, L.router, L.router_bias, x, n_tok, NE,
                           L.n_embd, L.top_k, W, fuse);
    else
        hipLaunchKernelGGL(k_route_logits<false>, grid, dim3(256), 0, s, L.router, L.router_bias, x, n_tok, NE,
                           L.n_embd, L.top_k, W, fuse);
    if (!fuse) {
        hipLaunchKernelGGL(k_topk, dim3((n_tok + 3) / 4), dim3(256), 0, s, n_tok, NE, L.top_k, W);
        hipLaunchKernelGGL(k_bucket, dim3(1), dim3(1024), 0, s, n_tok, NE, L.top_k, W);
    }
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
