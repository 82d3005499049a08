// decode.hip - the whole MoE block for one decode token in ONE persistent launch.
//
// Generation is bandwidth-bound ("ds4 深度实战...", section 5.1) and the pages
// fuse MoE routing with the expert computation into one GPU dispatch (same
// page, section 2.3).  Here one persistent launch walks a fixed list of work
// items in five phases, in this order:
//   router    : half an expert's logit per item (fp64 accumulation); a hash
//               layer scores only the k experts of the token's table row;
//   routing   : every workgroup polls until all router halves of this call
//               are stored and takes the top-k and renormalised weights itself
//               (the shared expert's first gate/up rows stream meanwhile);
//   shared g/u: one row of the shared expert's gate and up per wave;
//   routed g/u: 16 rows of one selected expert's IQ2 gate and up per item,
//               SiLU(g)*u kept in fp32;
//   routed dn : rows of one selected expert's Q2_K down projection, scaled
//               by its routing weight, from that slot's h vector in LDS;
//   shared dn : rows of the shared down projection.
// Items are dealt round-robin over the workgroups in phase order (routed down
// units in consecutive runs, so a workgroup's units mostly share one h
// vector), and the grid is sized to what the GPU holds at once (the occupancy
// query at create), so every wait is on data that a resident workgroup
// produces earlier in its own list and that never waits on a later one.  Each
// wait is also bounded (if the GPU is shared with other work, some workgroups
// may not be resident): if it ever expires, the workgroup
// records the call's tag in the host-visible status word, skips the work that
// depended on it and poisons the output with NaN instead of hanging.
//
// Hand-offs need no fences, counters or drains.  Every value another
// workgroup reads (the router half-sums, the h vectors) is stored as 64-bit
// words, each holding 32 bits of data under a 32-bit tag that identifies the
// call; a 64-bit store is seen whole or not at all.  Consumers poll the words
// with agent-scope loads (which read the device's point of coherence) until
// all of them carry this call's tag, and have the values in the same round
// trip.  Tags only change between calls, so nothing is reset.
// The block output (routed + shared) is added into the residual with fp32
// atomics.
#include "common.h"
#include "iq2_tables.h"

namespace ds4 {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ float dec_dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ float dec_silu(float z) { return z / (1.0f + expf(-z)); }


// Load at a 32-bit byte offset from a workgroup-uniform base.  Every plane
// read this way is below 4 GiB (the largest, an expert matrix plane, holds at
// most 256 x 4096 x 4096 / 4 bytes), and a zero-extended 32-bit offset lets
// the compiler keep the base in scalar registers and one offset per lane.
template <class T>
__device__ __forceinline__ T ld_at(const void *base, uint32_t off) {
    return *reinterpret_cast<const T *>(reinterpret_cast<const uint8_t *>(base) + off);
}
// Weights are read once per call: non-temporal loads (common.h).
template <typename T>
__device__ __forceinline__ T ld_nt(const void *base, uint32_t off);
template <>
__device__ __forceinline__ uint4 ld_nt<uint4>(const void *base, uint32_t off) {
    return ld_nt16(reinterpret_cast<const uint8_t *>(base) + off);
}
template <>
__device__ __forceinline__ uint32_t ld_nt<uint32_t>(const void *base, uint32_t off) {
    return ld_nt4(reinterpret_cast<const uint8_t *>(base) + off);
}
template <>
__device__ __forceinline__ uint16_t ld_nt<uint16_t>(const void *base, uint32_t off) {
    return ld_nt2(reinterpret_cast<const uint8_t *>(base) + off);
}

constexpr int DEC_WAVES = 4;
constexpr int DEC_THREADS = 64 * DEC_WAVES;
constexpr int DEC_WG_PER_CU = 2;  // resident workgroups per CU
constexpr int DEC_GU_NR = 4;  // routed gate/up row slots per wave
constexpr int DEC_DN_NR = 4;  // routed down row slots per wave

struct DecPlan {
    unsigned long long ep;  // calls already made on this workspace
    int n_route, n_shgu, n_rgu, n_shdn, n_rdn;   // n_route: 2 items per expert scored
    int rgu_per_slot, rdn_per_slot;
    int pre_routed;         // the routing is in W (idx, w, lists) from the router kernel: no router phase
    int shdn_cpr;
    int total;
};

// An agent-scope read of a tagged word (the device's point of coherence),
// as a global rather than a flat access.
__device__ __forceinline__ unsigned long long poll_load(const unsigned long long *p) {
    return __hip_atomic_load((const __attribute__((address_space(1))) unsigned long long *)p, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

// One tagged word: fp32 bits below, the call's tag above.  A 64-bit store is
// seen whole or not at all, so a reader that finds the tag has the value.
__device__ __forceinline__ void st_tagged(unsigned long long *p, float v, uint32_t tag) {
    __hip_atomic_store(p, ((unsigned long long)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- P0: router

// Routing of the token, computed by every workgroup for itself (wave 0) once
// all router halves are counted: fp32 logits from the fp64 halves, top-k with
// the lowest index first among equal logits, renormalised weights.  Workgroup
// 0 also writes it (and the per-expert lists) to the workspace for
// ds4moe_route's export.
struct RouteCache {
    int idx[MAX_TOPK];
    float w[MAX_TOPK];
    int slot[MAX_TOPK];  // where each selected expert's weights are (expert_slot)
};

// The weights and the export of a routing whose lane j < k holds slot j's
// expert and fp32 logit: one exp per lane (relative to the largest of the k
// logits, slot 0's for a top-k selection), the denominator by a sum over the
// k lanes.  set_experts: also record the experts in rc (a hash layer has them
// there already, and other waves may be reading them).
__device__ __forceinline__ void dec_route_finish(const Layer &L, const Work &W, int myE, float myL, RouteCache *rc,
                                                 bool write_global, bool set_experts = true) {
    const int lane = threadIdx.x & 63;
    const int NE = L.n_expert, k = L.top_k;
    float M = (lane < k) ? myL : -INFINITY;
    M = wave_max_dpp(M);
    const double ex = (lane < k) ? exp((double)myL - (double)M) : 0.0;
    const double z = wave_sum_dpp(ex);
    const float wj = (float)(ex / z);
    if (lane < k) {
        if (set_experts) {
            rc->idx[lane] = myE;
            rc->slot[lane] = expert_slot(L, myE);
        }
        rc->w[lane] = wj;
    }
    if (!write_global) return;
    if (lane < k) {
        W.idx[lane] = myE;
        W.w[lane] = wj;
    }
    int selE[MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MAX_TOPK; ++j) selE[j] = (j < k) ? __shfl(myE, j, 64) : 0;
    for (int ee = lane; ee <= NE; ee += 64) {
        int before = 0;
#pragma unroll
        for (int j = 0; j < MAX_TOPK; ++j)
            if (j < k) before += selE[j] < ee;
        W.offsets[ee] = before;
    }
    if (lane == 0) W.active[0] = k;
    if (lane < k) {
        int rank = 0;
#pragma unroll
        for (int i = 0; i < MAX_TOPK; ++i)
            if (i < k) rank += selE[i] < myE;
        W.active[1 + rank] = myE;
        W.list[rank] = lane;
    }
}

__device__ __forceinline__ void dec_topk_local(const Layer &L, const Work &W, const double *lg, RouteCache *rc,
                                               bool write_global) {
    const int lane = threadIdx.x & 63;
    const int NE = L.n_expert, k = L.top_k;
    // fp32 logits as order-preserving keys (0 = no expert); lane l holds
    // experts l + 64 i, whose fp64 logits (both halves and the bias) are lg[i]
    uint32_t key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) key[i] = lane + 64 * i < NE ? logit_key32((float)lg[i]) : 0u;
    // lane j < k ends up holding the j-th selection
    int myE = 0;
    float myL = 0.f;
#pragma unroll
    for (int j = 0; j < MAX_TOPK; ++j) {
        if (j >= k) break;
        uint32_t m;
        int ee;
        topk_round(key, m, ee);
        if (lane == j) myE = ee, myL = key32_logit(m);
    }
    dec_route_finish(L, W, myE, myL, rc, write_global);
}

// Half h of expert e's logit: waves split the half row (E/2 elements).
template <bool XBF16>
__device__ __forceinline__ void dec_route_item(const Layer &L, const Work &W, const void *__restrict__ x, int e,
                                               int h, double *lds_part, uint32_t tag) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int E = L.n_embd;
    const int half = E >> 1, per_wave = half >> 2;   // E/8 elements per wave
    const int base = h * half + wave * per_wave;
    double acc = 0.0;
    for (int i = 4 * lane; i < per_wave; i += 256) {
        const float4 r = ld_nt_f4(L.router + (int64_t)e * E + base + i);
        float4 xv;
        if (XBF16) {
            const uint2 v = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(x) + base + i);
            xv = make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                             __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
        } else {
            xv = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(x) + base + i);
        }
        acc = fma((double)xv.x, (double)r.x, acc);
        acc = fma((double)xv.y, (double)r.y, acc);
        acc = fma((double)xv.z, (double)r.z, acc);
        acc = fma((double)xv.w, (double)r.w, acc);
    }
    acc = wave_sum_dpp(acc);
    if (lane == 0) lds_part[wave] = acc;
    __syncthreads();
    if (threadIdx.x < 2) {
        // the half-sum's two 32-bit halves, each in one 64-bit store with the
        // call's tag above it: a reader that finds the tag has that half
        const double sum = lds_part[0] + lds_part[1] + lds_part[2] + lds_part[3];
        const unsigned long long bits = (unsigned long long)__double_as_longlong(sum);
        const unsigned long long part = threadIdx.x ? (bits >> 32) : (bits & 0xFFFFFFFFull);
        __hip_atomic_store(W.rtag + 4 * e + 2 * h + threadIdx.x, ((unsigned long long)tag << 32) | part,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------- P1: shared gate/up
// One shared gate/up item (one row of gate and up per wave): the weights and
// the matching x chunks (chunk ch = lane + 64 c, 8 elements each), as loaded.
template <bool XBF16>
struct ShguW {
    uint4 wg[8], wu[8];
    uint4 xv[XBF16 ? 8 : 16];
};
template <bool XBF16>
__device__ __forceinline__ void dec_shgu_load(const Layer &L, const void *__restrict__ x, int item, ShguW<XBF16> &w) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int E = L.n_embd, F = L.n_ff;
    const int nch = E >> 3;  // 16-byte chunks per row
    // rows past n_ff and chunks past the row read valid data that the
    // computation drops
    const int f = min(item * DEC_WAVES + wave, F - 1);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t ch = min(lane + 64 * c, nch - 1);
        w.wg[c] = ld_nt<uint4>(L.sh_gate, 2u * ((uint32_t)f * E + ch * 8u));
        w.wu[c] = ld_nt<uint4>(L.sh_up, 2u * ((uint32_t)f * E + ch * 8u));
        if (XBF16) {
            w.xv[c] = ld_at<uint4>(x, 16u * ch);
        } else {
            w.xv[2 * c] = ld_at<uint4>(x, 32u * ch);
            w.xv[2 * c + 1] = ld_at<uint4>(x, 32u * ch + 16u);
        }
    }
}
template <bool XBF16>
__device__ __forceinline__ void dec_shgu_compute(const Layer &L, const Work &W, int item, const ShguW<XBF16> &w,
                                                 uint32_t tag) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int E = L.n_embd, F = L.n_ff, k = L.top_k;
    const int nch = E >> 3;
    const int f = item * DEC_WAVES + wave;
    float g = 0.0f, u = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        if (lane + 64 * c < nch) {
            if (XBF16) {
                const uint4 xv = w.xv[c];
                g = dec_dot2(w.wg[c].x, xv.x, g), g = dec_dot2(w.wg[c].y, xv.y, g);
                g = dec_dot2(w.wg[c].z, xv.z, g), g = dec_dot2(w.wg[c].w, xv.w, g);
                u = dec_dot2(w.wu[c].x, xv.x, u), u = dec_dot2(w.wu[c].y, xv.y, u);
                u = dec_dot2(w.wu[c].z, xv.z, u), u = dec_dot2(w.wu[c].w, xv.w, u);
            } else {
                const uint4 a = w.xv[2 * c], b = w.xv[2 * c + 1];
                const float xf[8] = {__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z),
                                     __uint_as_float(a.w), __uint_as_float(b.x), __uint_as_float(b.y),
                                     __uint_as_float(b.z), __uint_as_float(b.w)};
                const uint32_t gw[4] = {w.wg[c].x, w.wg[c].y, w.wg[c].z, w.wg[c].w};
                const uint32_t uw[4] = {w.wu[c].x, w.wu[c].y, w.wu[c].z, w.wu[c].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    g = fmaf(__uint_as_float(gw[i] << 16), xf[2 * i], g);
                    g = fmaf(__uint_as_float(gw[i] & 0xFFFF0000u), xf[2 * i + 1], g);
                    u = fmaf(__uint_as_float(uw[i] << 16), xf[2 * i], u);
                    u = fmaf(__uint_as_float(uw[i] & 0xFFFF0000u), xf[2 * i + 1], u);
                }
            }
        }
    }
    g = wave_sum(g);
    u = wave_sum(u);
    if (lane == 0 && f < F) st_tagged(W.htag + (int64_t)k * F + f, dec_silu(g) * u, tag);
}

// ---------------------------------------------------------------- P2: routed gate/up (IQ2)
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
__device__ __forceinline__ float dec_dot2h(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}
__device__ __forceinline__ uint32_t dec_pack_f16(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

// The lane's 64 values of x (its column chunk of every routed gate/up row) as
// fp16 pairs, in registers for the whole phase, times 2^-k with k chosen from
// the chunk's largest magnitude so no value overflows fp16 (the partial dot
// products are scaled back by 2^k).  bf16 x converts exactly (fp16 has the
// longer mantissa) except below fp16's normal range, whose share of a dot
// product is under 2^-14 of the chunk's largest term; fp32 x is split into
// an fp16 high part and an fp16 low part, 22 bits in all.
template <bool XBF16>
struct DecX {
    static constexpr int NP = XBF16 ? 1 : 2;  // parts
    uint32_t v[NP][32];
    float scale;
    __device__ __forceinline__ void load(const void *x, int off) {
        float f[64];
        if (XBF16) {
            const uint4 *p = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(x) + off);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint4 r = p[i];
                const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    f[8 * i + 2 * q] = __uint_as_float(w[q] << 16);
                    f[8 * i + 2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
                }
            }
        } else {
            const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(x) + off);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float4 r = p[i];
                f[4 * i] = r.x, f[4 * i + 1] = r.y, f[4 * i + 2] = r.z, f[4 * i + 3] = r.w;
            }
        }
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < 64; ++i) mx = fmaxf(mx, fabsf(f[i]));
        // 2^-k with mx * 2^-k < 2^15
        const int ex = (int)((__float_as_uint(mx) >> 23) & 0xFFu) - 127;
        const int k = ex > 14 ? ex - 14 : 0;
        const float down = __uint_as_float((uint32_t)(127 - k) << 23);
        scale = __uint_as_float((uint32_t)(127 + k) << 23);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const float a = f[2 * i] * down, b = f[2 * i + 1] * down;
            v[0][i] = dec_pack_f16(a, b);
            if (!XBF16) {
                const float ah = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[0][i] & 0xFFFFu));
                const float bh = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[0][i] >> 16));
                v[NP - 1][i] = dec_pack_f16(a - ah, b - bh);
            }
        }
    }
    // 8 weights (4 fp16 pairs) of group grp8 against the matching x
    __device__ __forceinline__ float dot8(const uint4 &Lv, int grp8, float s) const {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            s = dec_dot2h(Lv.x, v[p][4 * grp8], s);
            s = dec_dot2h(Lv.y, v[p][4 * grp8 + 1], s);
            s = dec_dot2h(Lv.z, v[p][4 * grp8 + 2], s);
            s = dec_dot2h(Lv.w, v[p][4 * grp8 + 3], s);
        }
        return s;
    }
};

// One canonical IQ2 sub-block (32 weights: 4 codebook indices in word ib, 7
// sign bits per group of 8 and the 4-bit scale in word sw) of one lane.  The
// table lookups (TL / TS: level bytes and sign bytes, entry e, replica r at
// e * IQ2B_REPL + r) are issued one sub-block ahead of the arithmetic that
// uses them, so the LDS latency overlaps the previous sub-block's dot products.
struct Iq2Tab {
    uint2 lv[4], sv[4];
};
__device__ __forceinline__ void dec_iq2_fetch(const uint2 *TL, const uint2 *TS, uint32_t ib, uint32_t sw, int rep,
                                              Iq2Tab &t) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        t.lv[g] = TL[((ib >> (8 * g)) & 0xFFu) * IQ2B_REPL + rep];
        t.sv[g] = TS[((sw >> (7 * g)) & 0x7Fu) * IQ2B_REPL + rep];
    }
}
// The sub-block's dot product with x (x groups 4 sb .. 4 sb + 3 of the lane's
// chunk), times its odd scale 2 ls + 1; before d/64 and the lane's x scale.
// Two accumulators halve the chain of dependent dot products.
template <bool XBF16>
__device__ __forceinline__ float dec_iq2_sub(const Iq2Tab &t, uint32_t sw, const DecX<XBF16> &xc, int sb) {
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; g += 2) {
        s0 = xc.dot8(iq2_expand_f16(make_uint2(t.lv[g].x ^ t.sv[g].x, t.lv[g].y ^ t.sv[g].y)), 4 * sb + g, s0);
        s1 = xc.dot8(iq2_expand_f16(make_uint2(t.lv[g + 1].x ^ t.sv[g + 1].x, t.lv[g + 1].y ^ t.sv[g + 1].y)),
                     4 * sb + g + 1, s1);
    }
    return (float)(2u * (sw >> 28) + 1u) * (s0 + s1);
}

// Wait until every router half-sum of this call is stored, then route
// locally (wave 0).  Each lane polls the tagged words of its experts (l + 64 i)
// with agent-scope loads until all carry this call's tag: the values come
// with the tags, in one round trip once they are there.  Returns false if the
// bounded wait expired.
__device__ __forceinline__ void dec_route_poll(const Layer &L, const Work &W, uint32_t tag, RouteCache *rc,
                                               int *lds_flag) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x, NE = L.n_expert;
        float bias[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            bias[i] = L.router_bias ? L.router_bias[min(lane + 64 * i, NE - 1)] : 0.0f;
        unsigned long long v[4][4];
        uint32_t missing = 0;  // bit 4 i + q: word q of expert lane + 64 i not yet of this call
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v[i][q] = 0;
                if (lane + 64 * i < NE) missing |= 1u << (4 * i + q);
            }
        const uint32_t want = tag ^ W.want_xor;
        int spins = 0, ok = 1;
        while (true) {
            // all 16 words in flight at once (a word that already carries the
            // tag reads the same again), then the tags
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    v[i][q] = poll_load(W.rtag + 4 * min(lane + 64 * i, NE - 1) + q);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if ((uint32_t)(v[i][q] >> 32) == want) missing &= ~(1u << (4 * i + q));
            if (!__any(missing != 0)) break;
            __builtin_amdgcn_s_sleep(4);
            if (++spins > W.spin_limit) {
                if (lane == 0) report_wait_expired(W, tag);
                ok = 0;
                break;
            }
        }
        if (ok) {
            double lg[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const double h0 = __longlong_as_double((long long)((v[i][0] & 0xFFFFFFFFull) | (v[i][1] << 32)));
                const double h1 = __longlong_as_double((long long)((v[i][2] & 0xFFFFFFFFull) | (v[i][3] << 32)));
                lg[i] = h0 + h1 + (double)bias[i];
            }
            dec_topk_local(L, W, lg, rc, blockIdx.x == 0);
        }
        if (lane == 0) *lds_flag = ok;
    }
}

// The weights of a hash layer's token: lane j < k polls the four tagged
// words of slot j's expert (row `trow` of the table), then the weights are
// taken over those k logits.  The experts themselves are already in rc (set
// from the table row when the call starts).  A bad id (decided by every
// workgroup alike from the same word) skips the wait and fails the call.
__device__ __forceinline__ void dec_route_poll_hashed(const Layer &L, const Work &W, uint32_t tag,
                                                      const int32_t *trow, bool bad_id, RouteCache *rc,
                                                      int *lds_flag) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x, k = L.top_k;
        int ok = 1;
        if (bad_id) {
            if (lane == 0) report_bad_id(W, tag);
            ok = 0;
        } else {
            const int e = trow[min(lane, k - 1)];
            const float b = L.router_bias ? L.router_bias[e] : 0.0f;
            unsigned long long v[4] = {0, 0, 0, 0};
            uint32_t missing = lane < k ? 0xFu : 0u;
            const uint32_t want = tag ^ W.want_xor;
            int spins = 0;
            while (true) {
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = poll_load(W.rtag + 4 * e + q);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if ((uint32_t)(v[q] >> 32) == want) missing &= ~(1u << q);
                if (!__any(missing != 0)) break;
                __builtin_amdgcn_s_sleep(4);
                if (++spins > W.spin_limit) {
                    if (lane == 0) report_wait_expired(W, tag);
                    ok = 0;
                    break;
                }
            }
            if (ok) {
                const double h0 = __longlong_as_double((long long)((v[0] & 0xFFFFFFFFull) | (v[1] << 32)));
                const double h1 = __longlong_as_double((long long)((v[2] & 0xFFFFFFFFull) | (v[3] << 32)));
                dec_route_finish(L, W, e, (float)(h0 + h1 + (double)b), rc, blockIdx.x == 0, false);
            }
        }
        if (lane == 0) *lds_flag = ok;
    }
}

// Weights of one routed gate/up item for this lane: DEC_GU_NR rows of gate and
// up, with their fp16 scales d as loaded.  Nothing here looks at the loaded
// values: the item after the current one is loaded while the current one is
// computed, and any use of a value would wait for every load in flight.
struct RguW {
    uint4 qg[DEC_GU_NR], qu[DEC_GU_NR];
    uint32_t dg[DEC_GU_NR], du[DEC_GU_NR];
};

__device__ __forceinline__ void dec_rgu_load(const Layer &L, const DecPlan &P, const RouteCache *rc, int item,
                                             RguW &w) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int E = L.n_embd, F = L.n_ff;
    const int lpr = E >> 6, rpw = 64 / lpr;
    const int c = lane & (lpr - 1);
    const int j = item / P.rgu_per_slot, tile = item - j * P.rgu_per_slot;
    const int f0 = (tile * DEC_WAVES + wave) * (DEC_GU_NR * rpw) + lane / lpr;
    const int e = rc->slot[j];
#pragma unroll
    for (int r = 0; r < DEC_GU_NR; ++r) {
        // rows past n_ff (if any) read row n_ff - 1; the computation drops them
        const int f = f0 + r * rpw;
        const uint32_t rb = ((uint32_t)e * F + min(f, F - 1)) * L.nbe;
        w.qg[r] = ld_nt<uint4>(L.iq2_qs[0], rb * 64u + c * 16u);
        w.qu[r] = ld_nt<uint4>(L.iq2_qs[1], rb * 64u + c * 16u);
        w.dg[r] = ld_nt<uint16_t>(L.iq2_d[0], 2u * (rb + (c >> 2)));
        w.du[r] = ld_nt<uint16_t>(L.iq2_d[1], 2u * (rb + (c >> 2)));
    }
}

// Word pair (codebook indices, signs and scale) of sub-block n of an item's
// lane data: row n / 4, gate (n / 2 even) or up, canonical sub-block n % 2.
__device__ __forceinline__ uint2 dec_rgu_words(const RguW &w, int n) {
    const uint4 q = ((n >> 1) & 1) ? w.qu[n >> 2] : w.qg[n >> 2];
    return (n & 1) ? make_uint2(q.z, q.w) : make_uint2(q.x, q.y);
}

template <bool XBF16>
__device__ __forceinline__ void dec_rgu_compute(const Layer &L, const Work &W, const DecX<XBF16> &xc, const uint2 *TL,
                                                const uint2 *TS, int item, const DecPlan &P, const RguW &w,
                                                uint32_t tag) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int E = L.n_embd, F = L.n_ff;
    const int lpr = E >> 6, rpw = 64 / lpr;
    const int c = lane & (lpr - 1);
    const int j = item / P.rgu_per_slot, tile = item - j * P.rgu_per_slot;
    const int f0 = (tile * DEC_WAVES + wave) * (DEC_GU_NR * rpw) + lane / lpr;
    const int rep = lane & (IQ2B_REPL - 1);
    // sub-block n (of NS) is row n / 4, gate or up, canonical sub-block n % 2;
    // its lookups are issued while sub-block n - 1 is computed, into two named
    // buffers by parity (no selects between them), and each scheduling barrier
    // keeps the lookups after it (their registers) from being hoisted
    constexpr int NS = 4 * DEC_GU_NR;
    Iq2Tab t0, t1;
    {
        const uint2 q = dec_rgu_words(w, 0);
        dec_iq2_fetch(TL, TS, q.x, q.y, rep, t0);
    }
    float a[2];
#pragma unroll
    for (int n = 0; n < NS; n += 2) {
        {
            const uint2 q = dec_rgu_words(w, n + 1);
            dec_iq2_fetch(TL, TS, q.x, q.y, rep, t1);
        }
        a[(n >> 1) & 1] = dec_iq2_sub<XBF16>(t0, dec_rgu_words(w, n).y, xc, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (n + 2 < NS) {
            const uint2 q = dec_rgu_words(w, n + 2);
            dec_iq2_fetch(TL, TS, q.x, q.y, rep, t0);
        }
        a[(n >> 1) & 1] += dec_iq2_sub<XBF16>(t1, dec_rgu_words(w, n + 1).y, xc, 1);
        if ((n & 3) == 2) {
            // row r complete: gate in a[0], up in a[1], summed over the row's
            // lanes into its last one
            const int r = n >> 2, f = f0 + r * rpw;
            float g = a[0] * (half_to_f32((uint16_t)w.dg[r]) * xc.scale);
            float u = a[1] * (half_to_f32((uint16_t)w.du[r]) * xc.scale);
            g = group_sum_last(g, lpr) * 0.015625f;
            u = group_sum_last(u, lpr) * 0.015625f;
            if (c == lpr - 1 && f < F) st_tagged(W.htag + (int64_t)j * F + f, dec_silu(g) * u, tag);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ---------------------------------------------------------------- h vectors in LDS
// h vector float4 u (elements 4u .. 4u+3, in chunk c = u / 16) sits at slot
// 16 c + ((u % 16) ^ (c % 16)): the 16 lanes reading float4 i of their
// 64-element chunks hit 16 different bank quads, and so do lanes reading
// consecutive 8-element chunks.
__device__ __forceinline__ int h_slot(int u) { return (u & ~15) | ((u & 15) ^ ((u >> 4) & 15)); }

// Staging h vector `slot` of this call into H in two parts.  dec_h_issue
// loads the thread's tagged words (float4 u = thread + 256 q of h) early, so
// their round trip overlaps other work; dec_h_finish polls again whatever did
// not carry this call's tag yet, then stores the values.  dec_h_finish
// returns false, for the whole workgroup, if the bounded wait expired.
struct HPre {
    unsigned long long v[4][4];
};
__device__ __forceinline__ void dec_h_issue(const Work &W, int F, int slot, HPre &p) {
    const unsigned long long *src = W.htag + (int64_t)slot * F;
    const int n4 = F >> 2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        // past the vector: re-read its last float4, ignored below
        const int u = min((int)threadIdx.x + 256 * q, n4 - 1);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            p.v[q][e] = poll_load(src + 4 * u + e);
    }
}
__device__ __forceinline__ bool dec_h_finish(const Work &W, int F, int slot, uint32_t tag, float4 *H, HPre &p) {
    const unsigned long long *src = W.htag + (int64_t)slot * F;
    const int n4 = F >> 2;  // float4 of h
    const uint32_t want = tag ^ W.want_xor;
    // the previous item's reads of H are over
    __syncthreads();
    int ok = 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int u = threadIdx.x + 256 * q;
        if (ok && u < n4) {
            unsigned long long *v = p.v[q];
            uint32_t missing = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if ((uint32_t)(v[e] >> 32) != want) missing |= 1u << e;
            int spins = 0;
            while (missing) {
                __builtin_amdgcn_s_sleep(4);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = poll_load(src + 4 * u + e);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if ((uint32_t)(v[e] >> 32) == want) missing &= ~(1u << e);
                if (missing && ++spins > W.spin_limit) {
                    report_wait_expired(W, tag);
                    ok = 0;
                    break;
                }
            }
            if (ok)
                H[h_slot(u)] = make_float4(__uint_as_float((uint32_t)v[0]), __uint_as_float((uint32_t)v[1]),
                                           __uint_as_float((uint32_t)v[2]), __uint_as_float((uint32_t)v[3]));
        }
    }
    return __syncthreads_and(ok) != 0;
}

// ---------------------------------------------------------------- P3: shared down
// CPR = 16-byte chunks per lane per row (F / 512, at least 1); 16 chunk loads in
// flight per wave, i.e. 16 / CPR rows per wave.
template <int CPR>
__device__ __forceinline__ void dec_shdn_item(const Layer &L, const Work &W, float *__restrict__ out, int item, uint32_t tag,
                              float4 *H, int &hid, bool &ok) {
    constexpr int RPW = 16 / CPR;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int E = L.n_embd, F = L.n_ff, k = L.top_k;
    const int nch = F >> 3;
    const int r0 = (item * DEC_WAVES + wave) * RPW;
    // the shared h vector's words are requested first (when not staged yet),
    // then the weights (rows and chunks past the matrix read valid data that
    // is dropped below): the h round trip overlaps the weights' and its wait
    // does not include them
    const bool stage = hid != k;
    HPre hp;
    if (stage) dec_h_issue(W, F, k, hp);
    uint4 wv[RPW][CPR];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
        for (int c = 0; c < CPR; ++c) {
            const uint32_t row = min(r0 + rr, E - 1), ch = min(lane + 64 * c, nch - 1);
            wv[rr][c] = ld_nt<uint4>(L.sh_down, 2u * (row * F + ch * 8u));
        }
    // the shared h vector in LDS (its gate/up items, once all stored)
    if (stage) {
        if (!dec_h_finish(W, F, k, tag, H, hp)) {
            ok = false;
            return;
        }
        hid = k;
    }
    float hv[CPR][8];
#pragma unroll
    for (int c = 0; c < CPR; ++c) {
        const int ch = min(lane + 64 * c, nch - 1);
        const float4 a = H[h_slot(2 * ch)], b = H[h_slot(2 * ch + 1)];
        hv[c][0] = a.x, hv[c][1] = a.y, hv[c][2] = a.z, hv[c][3] = a.w;
        hv[c][4] = b.x, hv[c][5] = b.y, hv[c][6] = b.z, hv[c][7] = b.w;
    }
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
        float y = 0.0f;
#pragma unroll
        for (int c = 0; c < CPR; ++c) {
            if (lane + 64 * c >= nch) continue;
            const uint32_t a[4] = {wv[rr][c].x, wv[rr][c].y, wv[rr][c].z, wv[rr][c].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                y = fmaf(__uint_as_float(a[i] << 16), hv[c][2 * i], y);
                y = fmaf(__uint_as_float(a[i] & 0xFFFF0000u), hv[c][2 * i + 1], y);
            }
        }
        y = wave_sum(y);
        const int row = r0 + rr;
        if (lane == 0 && row < E) atomicAdd(out + row, y);
    }
}

// ---------------------------------------------------------------- P4: routed down (Q2_K)

// Weights of one routed down item for this lane: DEC_DN_NR rows.
struct RdnW {
    uint4 qs[DEC_DN_NR];
    uint32_t sc[DEC_DN_NR], dd[DEC_DN_NR];
};

__device__ __forceinline__ void dec_rdn_load(const Layer &L, const DecPlan &P, const RouteCache *rc, int item,
                                             RdnW &w) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int E = L.n_embd, F = L.n_ff;
    const int lpr = F >> 6, rpw = 64 / lpr;
    const int c = lane & (lpr - 1);
    const int j = item / P.rdn_per_slot, tile = item - j * P.rdn_per_slot;
    const int r0 = (tile * DEC_WAVES + wave) * (DEC_DN_NR * rpw) + lane / lpr;
    const int e = rc->slot[j];
#pragma unroll
    for (int r = 0; r < DEC_DN_NR; ++r) {
        // rows past n_embd (if any) read row n_embd - 1; the computation drops them
        const int row = r0 + r * rpw;
        const uint32_t rb = ((uint32_t)e * E + min(row, E - 1)) * L.nbf;
        w.qs[r] = ld_nt<uint4>(L.q2k_qs, rb * 64u + c * 16u);
        w.sc[r] = ld_nt<uint32_t>(L.q2k_sc, rb * 16u + c * 4u);
        w.dd[r] = ld_nt<uint32_t>(L.q2k_dd, 4u * (rb + (c >> 2)));
    }
}

// A routed slot's h vector staged in LDS for the Q2_K down projections, as
// fp16 pairs laid out for the reading lanes.  Lane chunk c (h[64 c .. 64 c +
// 63]) has per sub-block s (16 values, weight 4 b + u at bits 2u of byte b of
// the sub-block's qs word) two 16-byte units, one per byte pair k = b / 2:
// unit (2 s + k) * lpr + c holds, for u = 0..3, the pair
// (h[64 c + 16 s + 8 k + u], h[64 c + 16 s + 8 k + 4 + u]) * 2^-e_c * 4^-u.
// The 4^-u matches the weights, which enter the dot products as fp16
// subnormals q * 4^u * 2^-24 (the byte masked in place: no shifts, no offset
// to subtract); e_c puts the chunk's largest value in [2^14, 2^15), and
// Hsc[c] = 2^(24 + e_c) undoes both.  Hsum[s * lpr + c] is the sub-block's
// plain fp32 sum of h, for the min term.  Consecutive lanes read consecutive
// units: no bank conflicts.
// In two parts: dec_h16_issue loads the thread's tagged words early, so
// their round trip overlaps other loads issued after them; dec_h16_finish
// polls again whatever did not carry this call's tag yet, converts and
// stores.  dec_h16_finish returns false, for the whole workgroup, if the
// bounded wait expired.
struct H16Pre {
    unsigned long long v[2][8];
};
__device__ __forceinline__ void dec_h16_issue(const Work &W, int F, int slot, H16Pre &pre) {
    const unsigned long long *src = W.htag + (int64_t)slot * F;
    const int np = F >> 3;  // thread steps of 8 values
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        // past the vector: re-read its last 8 values, ignored below
        const int p = min((int)threadIdx.x + 256 * q, np - 1);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            pre.v[q][e] = poll_load(src + 8 * p + e);
    }
}
__device__ __forceinline__ bool dec_h16_finish(const Work &W, int F, int slot, uint32_t tag, uint4 *Hq, float *Hsc,
                                               float *Hsum, H16Pre &pre) {
    const unsigned long long *src = W.htag + (int64_t)slot * F;
    const int np = F >> 3, lpr = F >> 6;  // thread steps of 8 values; lanes per row
    unsigned long long (&v)[2][8] = pre.v;
    const uint32_t want = tag ^ W.want_xor;
    // the previous unit's reads of the staged vector are over
    __syncthreads();
    int ok = 1;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int p = threadIdx.x + 256 * q;
        if (256 * q >= np) break;  // uniform
        const bool mine = p < np;  // np is a multiple of 32: whole groups of 8 lanes agree
        uint32_t missing = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (mine && (uint32_t)(v[q][e] >> 32) != want) missing |= 1u << e;
        int spins = 0;
        while (ok && missing) {
            __builtin_amdgcn_s_sleep(4);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[q][e] = poll_load(src + 8 * p + e);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if ((uint32_t)(v[q][e] >> 32) == want) missing &= ~(1u << e);
            if (missing && ++spins > W.spin_limit) {
                report_wait_expired(W, tag);
                ok = 0;
            }
        }
        float h[8];
        float mx = 0.0f, hs = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            h[e] = __uint_as_float((uint32_t)v[q][e]);
            mx = fmaxf(mx, fabsf(h[e]));
            hs += h[e];
        }
        // chunk c = p / 8 is 8 consecutive lanes; sub-block s = (p / 2) % 4 is 2.
        // By DPP (no LDS round trip): lane pairs, quad halves, then each lane
        // with its mirror in the other quad of the 8
        mx = fmaxf(mx, dpp_f32<0xB1, 0xF, false>(mx));   // quad_perm [1,0,3,2]
        mx = fmaxf(mx, dpp_f32<0x4E, 0xF, false>(mx));   // quad_perm [2,3,0,1]
        mx = fmaxf(mx, dpp_f32<0x141, 0xF, false>(mx));  // row_half_mirror
        hs += dpp_f32<0xB1, 0xF, false>(hs);
        if (mine) {
            const int ex = (int)((__float_as_uint(mx) >> 23) & 0xFFu) - 127;
            const int e = min(max(ex - 14, -100), 100);
            uint32_t pr[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                // 2^-e * 4^-u, exact
                const float down = __uint_as_float((uint32_t)(127 - e - 2 * u) << 23);
                pr[u] = dec_pack_f16(h[u] * down, h[4 + u] * down);
            }
            Hq[(p & 7) * lpr + (p >> 3)] = make_uint4(pr[0], pr[1], pr[2], pr[3]);
            if ((p & 7) == 0) Hsc[p >> 3] = __uint_as_float((uint32_t)(127 + 24 + e) << 23);
            if ((p & 1) == 0) Hsum[((p >> 1) & 3) * lpr + (p >> 3)] = hs;
        }
    }
    return __syncthreads_and(ok) != 0;
}
// Both parts at once.
__device__ __forceinline__ bool dec_stage_h16(const Work &W, int F, int slot, uint32_t tag, uint4 *Hq, float *Hsc,
                                              float *Hsum) {
    H16Pre pre;
    dec_h16_issue(W, F, slot, pre);
    return dec_h16_finish(W, F, slot, tag, Hq, Hsc, Hsum, pre);
}

// One routed down unit from the staged h vector: each Q2_K row of the lane (64
// weights: 4 sub-blocks of 16) is d * sum_s sc_s dot_s - dmin * sum_s m_s hsum_s.
// The 2-bit codes of byte pair k become fp16 pairs by one byte permute (bytes
// 2k, 2k+1 into the low bytes of the two halves) and, per position u, one mask
// (bits 2u, 2u+1 of each low byte): the subnormal q * 4^u * 2^-24, whose
// product with the staged h * 2^-e * 4^-u would be exact.  The dot product
// instruction does not keep it so on gfx950: with one subnormal operand a
// probe found results off by up to 3.1e-4 relative (normal operands: at most
// one fp32 ulp), an error of the same order as h's fp16 rounding.
__device__ __forceinline__ void dec_rdn_compute16(const Layer &L, float *__restrict__ out, int item, const DecPlan &P,
                                                  const RouteCache *rc, const RdnW &w, const uint4 *Hq,
                                                  const float *Hsc, const float *Hsum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int E = L.n_embd, F = L.n_ff;
    const int lpr = F >> 6, rpw = 64 / lpr;
    const int c = lane & (lpr - 1);
    const int j = item / P.rdn_per_slot, tile = item - j * P.rdn_per_slot;
    const int r0 = (tile * DEC_WAVES + wave) * (DEC_DN_NR * rpw) + lane / lpr;
    const float wgt = rc->w[j];
    const float hsc = Hsc[c];
    float A[DEC_DN_NR], B[DEC_DN_NR];
#pragma unroll
    for (int r = 0; r < DEC_DN_NR; ++r) A[r] = 0.0f, B[r] = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint4 h0 = Hq[(2 * s) * lpr + c], h1 = Hq[(2 * s + 1) * lpr + c];
        const float hsum = Hsum[s * lpr + c];
#pragma unroll
        for (int r = 0; r < DEC_DN_NR; ++r) {
            const uint32_t Q = s == 0 ? w.qs[r].x : s == 1 ? w.qs[r].y : s == 2 ? w.qs[r].z : w.qs[r].w;
            const uint32_t P0 = __builtin_amdgcn_perm(0u, Q, 0x0C010C00u);  // bytes 0, 1
            const uint32_t P1 = __builtin_amdgcn_perm(0u, Q, 0x0C030C02u);  // bytes 2, 3
            float d0 = 0.0f, d1 = 0.0f;
            d0 = dec_dot2h(P0 & 0x00030003u, h0.x, d0);
            d1 = dec_dot2h(P1 & 0x00030003u, h1.x, d1);
            d0 = dec_dot2h(P0 & 0x000C000Cu, h0.y, d0);
            d1 = dec_dot2h(P1 & 0x000C000Cu, h1.y, d1);
            d0 = dec_dot2h(P0 & 0x00300030u, h0.z, d0);
            d1 = dec_dot2h(P1 & 0x00300030u, h1.z, d1);
            d0 = dec_dot2h(P0 & 0x00C000C0u, h0.w, d0);
            d1 = dec_dot2h(P1 & 0x00C000C0u, h1.w, d1);
            const uint32_t scb = (w.sc[r] >> (8 * s)) & 0xFFu;
            A[r] = fmaf((float)(scb & 15u), d0 + d1, A[r]);
            B[r] = fmaf((float)(scb >> 4), hsum, B[r]);
        }
    }
#pragma unroll
    for (int r = 0; r < DEC_DN_NR; ++r) {
        const int row = r0 + r * rpw;
        const uint32_t dd = w.dd[r];
        float y = half_to_f32((uint16_t)(dd & 0xFFFFu)) * (A[r] * hsc) - half_to_f32((uint16_t)(dd >> 16)) * B[r];
        y = group_sum_last(y, lpr);
        if (c == lpr - 1 && row < E) atomicAdd(out + row, wgt * y);
    }
}

// Routed down items are handed out so that each workgroup's units are
// consecutive (slot-major), so they mostly share one h vector: local item
// l = G m + o (o < G) is unit o q + min(o, r) + m, with n = q G + r units.
__device__ __forceinline__ int dec_rdn_unit(int l, int G, int n) {
    const int o = l % G, q = n / G, r = n % G;
    return o * q + min(o, r) + l / G;
}

// ---------------------------------------------------------------- the persistent kernel
template <bool XBF16>
__global__ __launch_bounds__(DEC_THREADS, DEC_WG_PER_CU) void k_decode_fused(Layer L, Work W, const void *__restrict__ x,
                                                             float *__restrict__ out, DecPlan P) {
    __shared__ uint2 TL[256 * IQ2B_REPL];  // level bytes per codebook entry
    __shared__ uint2 TS[128 * IQ2B_REPL];  // sign bytes per pattern of 7 stored signs
    __shared__ int lds_flag;
    __shared__ double lds_part[DEC_WAVES];
    __shared__ RouteCache rc;
    __shared__ float4 H[1024];             // the shared h vector (n_ff <= 4096) for the shared down projection
    __shared__ uint4 Hq[512];              // a routed h vector as fp16 pairs (n_ff <= 4096)
    __shared__ float Hsc[64], Hsum[256];   // its per-chunk scales and per-sub-block sums
    const int G = gridDim.x;
    // item order: router, shared gate/up, routed gate/up, shared down, routed
    // down; every wait is on an earlier phase.  Shared down comes before routed
    // down so that the workgroups with one routed gate/up item (fewer than the
    // others) stream it while the others are still decoding IQ2 weights.
    const int b0 = P.n_route, b1 = b0 + P.n_shgu, b2 = b1 + P.n_rgu, b3 = b2 + P.n_shdn, b4 = b3 + P.n_rdn;
    // one loop per phase (the same items in the same order as a single loop
    // over all of them), so that each phase's registers are allocated on their own
    // loads that depend on nothing are issued before the router item: this
    // thread's codebook entry and the lane's slice of x for the routed gate/up
    // (lane c of a routed gate/up row holds x[64 c .. 64 c + 63])
    const uint32_t cb = L.codebook[threadIdx.x & 255];
    DecX<XBF16> xc;
    xc.load(x, 64 * ((threadIdx.x & 63) & ((L.n_embd >> 6) - 1)));
    int it = blockIdx.x;
    const uint32_t tag = (uint32_t)(P.ep % 0xFFFFFFFFull) + 1u;  // never 0, the workspace's initial value
    // a hash layer scores only the k experts of the token's table row
    const bool hashed = L.hash_table != nullptr;
    const int id = hashed ? W.ids[0] : 0;
    const bool bad_id = hashed && (id < 0 || id >= L.n_vocab);
    const int32_t *trow = hashed ? L.hash_table + (int64_t)(bad_id ? 0 : id) * L.top_k : nullptr;
    for (; it < b0; it += G) dec_route_item<XBF16>(L, W, x, hashed ? trow[it >> 1] : it >> 1, it & 1, lds_part, tag);
    // the IQ2 byte tables (entry e, replica r at e * IQ2B_REPL + r)
    {
        static_assert(DEC_THREADS == 256, "one codebook entry per thread");
        const uint2 ent = iq2_level_bytes(cb);
#pragma unroll
        for (int r = 0; r < IQ2B_REPL; ++r)
            TL[threadIdx.x * IQ2B_REPL + ((r + threadIdx.x) & (IQ2B_REPL - 1))] = ent;
        if (threadIdx.x < 128) {
            const uint2 sg = iq2_sign_bytes(threadIdx.x);
#pragma unroll
            for (int r = 0; r < IQ2B_REPL; ++r)
                TS[threadIdx.x * IQ2B_REPL + ((r + threadIdx.x) & (IQ2B_REPL - 1))] = sg;
        }
    }
    __syncthreads();
    // the first shared gate/up item's weights stream while the routing is
    // polled (the polls' round trip ends once they are in); then the first
    // routed gate/up item's weights stream while the shared items are computed
    // (wave 0 polls first and loads its row after: its polls do not queue
    // behind its own weights)
    ShguW<XBF16> sg;
    const bool wave0 = threadIdx.x < 64;
    if (!wave0 && it < b1) dec_shgu_load<XBF16>(L, x, it - b0, sg);
    if (P.pre_routed) {
        // routed by the router kernel earlier on the stream (host-resident
        // experts: the cache step ran in between and placed them)
        if (threadIdx.x < L.top_k) {
            const int ex = W.idx[threadIdx.x];
            rc.idx[threadIdx.x] = ex;
            rc.w[threadIdx.x] = W.w[threadIdx.x];
            rc.slot[threadIdx.x] = expert_slot(L, ex);
        }
        if (threadIdx.x == 0) lds_flag = 1;
    } else if (hashed) {
        // a hash layer's experts are its table row's, known at once: routed
        // gate/up starts without waiting for the logits, which set only the
        // weights and are polled before routed down (below)
        if (threadIdx.x < 64) {
            const int lane = threadIdx.x;
            if (!bad_id && lane < L.top_k) {
                const int e = trow[lane];
                rc.idx[lane] = e;
                rc.slot[lane] = expert_slot(L, e);
            }
            if (lane == 0) {
                if (bad_id) report_bad_id(W, tag);
                lds_flag = bad_id ? 0 : 1;
            }
        }
    } else {
        dec_route_poll(L, W, tag, &rc, &lds_flag);
    }
    if (wave0 && it < b1) dec_shgu_load<XBF16>(L, x, it - b0, sg);
    __syncthreads();
    bool ok = lds_flag != 0;
    __syncthreads();
    int it_r = it;
    while (it_r < b1) it_r += G;
    RguW wa, wb;   // two named buffers, alternating (no copies)
    if (ok && it_r < b2) dec_rgu_load(L, P, &rc, it_r - b1, wa);
    for (bool first = true; it < b1; it += G, first = false) {
        if (!first) dec_shgu_load<XBF16>(L, x, it - b0, sg);
        dec_shgu_compute<XBF16>(L, W, it - b0, sg, tag);
    }
    // routed gate/up: the next item's weights are in flight while this one is
    // computed.  A workgroup's last item runs at a raised wave priority: the
    // two workgroups of a CU share its SIMDs, the older one's waves win equal
    // priority, and the younger one (one item fewer) would otherwise wait for
    // both of the older one's items, delaying the slots later units need.
    if (ok && it < b2) {
        for (;;) {
            bool more = it + G < b2;
            if (more) dec_rgu_load(L, P, &rc, it + G - b1, wb);
            if (!more) __builtin_amdgcn_s_setprio(1);
            dec_rgu_compute<XBF16>(L, W, xc, TL, TS, it - b1, P, wa, tag);
            it += G;
            if (!more) break;
            more = it + G < b2;
            if (more) dec_rgu_load(L, P, &rc, it + G - b1, wa);
            if (!more) __builtin_amdgcn_s_setprio(1);
            dec_rgu_compute<XBF16>(L, W, xc, TL, TS, it - b1, P, wb, tag);
            it += G;
            if (!more) break;
        }
        __builtin_amdgcn_s_setprio(0);
    }
    int hid = -1;  // the h vector H holds (slot, or top_k for the shared one)
    for (; ok && it < b3; it += G) {
        switch (P.shdn_cpr) {
            case 1: dec_shdn_item<1>(L, W, out, it - b2, tag, H, hid, ok); break;
            case 2: dec_shdn_item<2>(L, W, out, it - b2, tag, H, hid, ok); break;
            case 4: dec_shdn_item<4>(L, W, out, it - b2, tag, H, hid, ok); break;
            default: dec_shdn_item<8>(L, W, out, it - b2, tag, H, hid, ok); break;
        }
    }
    // a hash layer's weights: wave 0 polls the k experts' logits (long since
    // written by the router items); every workgroup with routed down units
    // needs them, and workgroup 0 also exports the routing
    if (hashed && !P.pre_routed) {
        const bool poll = ok && (it < b4 || blockIdx.x == 0);
        if (poll) dec_route_poll_hashed(L, W, tag, trow, false, &rc, &lds_flag);
        __syncthreads();
        if (poll) ok = lds_flag != 0;
    }
    // routed down: each workgroup takes consecutive units (slot-major), so
    // its units mostly share one h vector, staged in LDS when the slot
    // changes (before the next unit's prefetch, so the staging's polls do not
    // wait for it); pipelined like routed gate/up otherwise
    if (ok && it < b4) {
        RdnW da, db;
        {
            // the first unit's h vector (H holds no routed one yet): its words
            // are requested before the unit's weights
            const int u = dec_rdn_unit(it - b3, G, P.n_rdn);
            hid = u / P.rdn_per_slot;
            H16Pre hp;
            dec_h16_issue(W, L.n_ff, hid, hp);
            dec_rdn_load(L, P, &rc, u, da);
            ok = dec_h16_finish(W, L.n_ff, hid, tag, Hq, Hsc, Hsum, hp);
        }
        for (; ok;) {
            int u = dec_rdn_unit(it - b3, G, P.n_rdn);
            if (u / P.rdn_per_slot != hid) {
                hid = u / P.rdn_per_slot;
                if (!(ok = dec_stage_h16(W, L.n_ff, hid, tag, Hq, Hsc, Hsum))) break;
            }
            bool more = it + G < b4;
            if (more) dec_rdn_load(L, P, &rc, dec_rdn_unit(it + G - b3, G, P.n_rdn), db);
            dec_rdn_compute16(L, out, u, P, &rc, da, Hq, Hsc, Hsum);
            it += G;
            if (!more) break;
            u = dec_rdn_unit(it - b3, G, P.n_rdn);
            if (u / P.rdn_per_slot != hid) {
                hid = u / P.rdn_per_slot;
                if (!(ok = dec_stage_h16(W, L.n_ff, hid, tag, Hq, Hsc, Hsum))) break;
            }
            more = it + G < b4;
            if (more) dec_rdn_load(L, P, &rc, dec_rdn_unit(it + G - b3, G, P.n_rdn), da);
            dec_rdn_compute16(L, out, u, P, &rc, db, Hq, Hsc, Hsum);
            it += G;
            if (!more) break;
        }
    }
    // a bounded wait of this workgroup expired, or the token's id is out of
    // range (either was reported for the host): the call's output is poisoned too.  An exchange at the device's point of
    // coherence, where the other contributions are added: whatever lands
    // before or after it, out[0] ends as NaN.
    if (!ok && threadIdx.x == 0) atomicExch(out, __builtin_nanf(""));
}

static DecPlan make_plan(const Layer &L) {
    DecPlan P{};
    const int E = L.n_embd, F = L.n_ff, k = L.top_k;
    // half an expert row per item: every expert, or the k of a hash layer's table row
    P.n_route = 2 * (L.hash_table ? L.top_k : L.n_expert);
    P.pre_routed = 0;
    P.n_shgu = L.n_shared ? (F + DEC_WAVES - 1) / DEC_WAVES : 0;
    const int rows_gu_item = DEC_WAVES * DEC_GU_NR * (64 / (E >> 6));
    P.rgu_per_slot = (F + rows_gu_item - 1) / rows_gu_item;
    P.n_rgu = k * P.rgu_per_slot;
    P.shdn_cpr = ((F >> 3) + 63) >> 6;
    const int rows_sd_item = DEC_WAVES * (16 / P.shdn_cpr);
    P.n_shdn = L.n_shared ? (E + rows_sd_item - 1) / rows_sd_item : 0;
    const int rows_dn_item = DEC_WAVES * DEC_DN_NR * (64 / (F >> 6));
    P.rdn_per_slot = (E + rows_dn_item - 1) / rows_dn_item;
    P.n_rdn = k * P.rdn_per_slot;
    P.total = P.n_route + P.n_shgu + P.n_rgu + P.n_shdn + P.n_rdn;
    return P;
}

int decode_grid(int act_bf16) {
    int dev = 0, ncu = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    hipError_t e;
    if (act_bf16)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(&k_decode_fused<true>),
                                                     DEC_THREADS, 0);
    else
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(&k_decode_fused<false>),
                                                     DEC_THREADS, 0);
    if (e != hipSuccess) return 0;
    per_cu = per_cu < 1 ? 1 : (per_cu > DEC_WG_PER_CU ? DEC_WG_PER_CU : per_cu);
    return ncu * per_cu;
}

hipError_t launch_decode_fused(const Layer &L, const Work &W, const void *x, float *out, int grid,
                               unsigned long long ep, hipStream_t s, bool pre_routed) {
    DecPlan P = make_plan(L);
    P.ep = ep;
    if (pre_routed) {
        P.pre_routed = 1;
        P.total -= P.n_route;
        P.n_route = 0;
    }
    Layer Lc = L;
    Work Wc = W;
    const void *xc = x;
    float *oc = out;
    void *args[] = {&Lc, &Wc, &xc, &oc, &P};
    const void *fn = (L.act_dtype == 1) ? reinterpret_cast<const void *>(&k_decode_fused<true>)
                                        : reinterpret_cast<const void *>(&k_decode_fused<false>);
    // A plain launch: a cooperative one (which would refuse a grid that cannot
    // be resident at once) measured 51.4 against 32.7 us per token.  The grid
    // is sized by the occupancy query at create, and every wait is bounded.
    hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(DEC_THREADS), args, 0, s);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace ds4
