// decode.hip - the whole MoE block for one decode token in ONE persistent launch.
//
// Generation is bandwidth-bound ("ds4 深度实战...", section 5.1) and the pages
// fuse MoE routing with the expert computation into one GPU dispatch (same
// page, section 2.3).  Here one persistent launch walks a fixed list of work
// items in five phases, in this order:
//   router    : half an expert's logit per item (fp64 accumulation);
//   shared g/u: 4 rows of the shared expert's gate and up per item (no
//               routing needed, so it streams while the router is counted);
//   routing   : every workgroup waits until all router halves are counted and
//               takes the top-k and renormalised weights itself;
//   routed g/u: 16 rows of one selected expert's IQ2 gate and up per item,
//               SiLU(g)*u kept in fp32;
//   routed dn : rows of one selected expert's Q2_K down projection, scaled
//               by its routing weight (waits for that expert's g/u items);
//   shared dn : rows of the shared down projection (waits for shared g/u).
// Items are dealt round-robin over the workgroups in phase order, and the grid
// is sized to what the GPU holds at once, so every wait is on an item that a
// resident workgroup took earlier and that never waits on a later one.  Each
// wait is also bounded: if it ever expires (the GPU shared with other work),
// the kernel poisons the output with NaN instead of hanging.
//
// Hand-offs avoid cache-maintenance fences (an L2 write-back or invalidate per
// hand-off costs more than the whole block).  Data another workgroup will read
// (logits, routing, the h vectors) is written with agent-scope stores, which
// write through to the device's point of coherence; the producer waits for
// its stores to complete and then bumps a counter with an agent-scope atomic.
// Consumers poll the counter with agent-scope loads and then read the data
// with plain loads: no workgroup touches those lines earlier in the launch and
// caches are invalidated between launches, so no stale copy can be hit.  The
// counters hold 64-bit epochs and never need resetting.
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
__device__ __forceinline__ float dec_group_sum(float v, int lpr) {
    for (int off = lpr >> 1; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Phase counters: 64-bit, each in its own 256-byte slot of W.counters (slot 0
// belongs to the multi-kernel router).  They only ever increase: call number
// `ep` of a handle waits for (ep + 1) times the per-call count, so nothing has
// to be reset at the end of a launch.
constexpr int CSTRIDE = 32;  // in uint64
constexpr int C_ROUTE = 1, C_SHGU = 3, C_ERR = 4, C_GU = 5;  // C_GU + slot; slot units
__device__ __forceinline__ unsigned long long *ctr(const Work &W, int slot) {
    return reinterpret_cast<unsigned long long *>(W.counters) + slot * CSTRIDE;
}

constexpr int DEC_WAVES = 4;
constexpr int DEC_THREADS = 64 * DEC_WAVES;
constexpr int DEC_WG_PER_CU = 2;  // resident workgroups per CU
constexpr int DEC_GU_NR = 4;  // routed gate/up row slots per wave
constexpr int DEC_DN_NR = 4;  // routed down row slots per wave

struct DecPlan {
    unsigned long long ep;  // calls already made on this workspace
    int n_route, n_shgu, n_rgu, n_shdn, n_rdn;
    int rgu_per_slot, rdn_per_slot;
    int shdn_cpr;
    int total;
};

constexpr int SPIN_LIMIT = 1 << 20;      // polls before giving up (about a second)

// Loads of data produced by other workgroups in this launch (small items).
__device__ __forceinline__ float ld_shared(const float *p) {
    return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t *>(p), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ int ld_shared(const int *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Store that other workgroups (any XCD) can read after the hand-off.
__device__ __forceinline__ void st_shared(float *p, float v) {
    __hip_atomic_store(reinterpret_cast<uint32_t *>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_shared(int *p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// This wavefront's shared stores are complete.
__device__ __forceinline__ void stores_done() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// The workgroup's shared stores are complete; then count the item (once).
// Returns the counter value before the increment (valid in thread 0).
__device__ __forceinline__ unsigned long long publish_item(unsigned long long *c) {
    stores_done();
    __syncthreads();
    unsigned long long prev = 0;
    if (threadIdx.x == 0) prev = __hip_atomic_fetch_add(c, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return prev;
}

// Wait (one poller per workgroup, with backoff) until *c >= target.  Returns
// false, and flags the error, if the bounded wait expired.
template <int SLEEP = 8>
__device__ __forceinline__ bool wait_items(const Work &W, unsigned long long *c, unsigned long long target,
                                           int *lds_flag) {
    if (threadIdx.x == 0) {
        int ok = 1, spins = 0;
        while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            __builtin_amdgcn_s_sleep(SLEEP);
            if (++spins > SPIN_LIMIT) {
                __hip_atomic_store(ctr(W, C_ERR), 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = 0;
                break;
            }
        }
        *lds_flag = ok;
    }
    __syncthreads();
    const bool ok = *lds_flag != 0;
    __syncthreads();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    return ok;
}


// ---------------------------------------------------------------- P0: router
// Each router item is half an expert row (the two halves land in separate
// fp64 slots of W.hbuf's router area, so nothing has to be cleared between
// calls).  The wavefront that completes the last half rounds every logit to
// fp32, takes the top-k with its renormalised weights, publishes "route
// ready", and only then writes the per-expert lists kept for ds4moe_route.
// Wave-wide maximum of an unsigned key by DPP (row shifts, then the two row
// broadcasts); the result is read from the last lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true));  // row_shr:1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true));  // row_shr:2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true));  // row_shr:4
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true));  // row_shr:8
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false)); // row_bcast:15
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false)); // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Routing of the token, computed by every workgroup for itself (wave 0) once
// all router halves are counted: fp32 logits from the fp64 halves, top-k with
// the lowest index first among equal logits, renormalised weights.  Workgroup
// 0 also writes it (and the per-expert lists) to the workspace for
// ds4moe_route's export.
struct RouteCache {
    int idx[MAX_TOPK];
    float w[MAX_TOPK];
};

__device__ __forceinline__ void dec_topk_local(const Layer &L, const Work &W, const double *part, RouteCache *rc,
                                               bool write_global) {
    const int lane = threadIdx.x & 63;
    const int NE = L.n_expert, k = L.top_k;
    // fp32 logits as order-preserving keys (0 = no expert); lane l holds experts l + 64 i.
    // The halves were stored by other workgroups with write-through stores and
    // no workgroup reads those lines before the count is complete: plain loads
    // are coherent.
    uint32_t key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ee = lane + 64 * i;
        key[i] = 0u;
        if (ee < NE) {
            const double2 hh = *reinterpret_cast<const double2 *>(part + 2 * ee);
            const float Lf = (float)(hh.x + hh.y + (L.router_bias ? (double)L.router_bias[ee] : 0.0));
            const uint32_t u = __float_as_uint(Lf);
            key[i] = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
            if (key[i] == 0u) key[i] = 1u;  // keep 0 free for "taken"
        }
    }
    // lane j < k ends up holding the j-th selection
    int myE = 0;
    float myL = 0.f;
#pragma unroll
    for (int j = 0; j < MAX_TOPK; ++j) {
        if (j >= k) break;
        const uint32_t m = wave_max_u32(max(max(key[0], key[1]), max(key[2], key[3])));
        int ee = -1;
#pragma unroll
        for (int i = 3; i >= 0; --i) {
            const uint64_t bb = __ballot(key[i] == m);
            if (bb) ee = 64 * i + (__ffsll((unsigned long long)bb) - 1);
        }
        const uint32_t u = (m & 0x80000000u) ? (m & 0x7FFFFFFFu) : ~m;
        if (lane == j) myE = ee, myL = __uint_as_float(u);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (lane + 64 * i == ee) key[i] = 0u;
    }
    // one exp per lane, the denominator by a sum over the k lanes
    const float L0 = __shfl(myL, 0, 64);
    const double ex = (lane < k) ? exp((double)myL - (double)L0) : 0.0;
    const double z = wave_sum(ex);
    const float wj = (float)(ex / z);
    if (lane < k) {
        rc->idx[lane] = myE;
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

// Half h of expert e's logit: waves split the half row (E/2 elements).
template <bool XBF16>
__device__ void dec_route_item(const Layer &L, const Work &W, const void *__restrict__ x, int item, int *lds_flag,
                               double *lds_part, const DecPlan &P) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int E = L.n_embd;
    const int e = item >> 1, h = item & 1;
    double *part = W.rhalf;
    const int half = E >> 1, per_wave = half >> 2;   // E/8 elements per wave
    const int base = h * half + wave * per_wave;
    double acc = 0.0;
    for (int i = 4 * lane; i < per_wave; i += 256) {
        const float4 r = *reinterpret_cast<const float4 *>(L.router + (int64_t)e * E + base + i);
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
    acc = wave_sum(acc);
    if (lane == 0) lds_part[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        const double sum = lds_part[0] + lds_part[1] + lds_part[2] + lds_part[3];
        __hip_atomic_store(part + 2 * e + h, sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // count the half (the increment's result is not needed)
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr(W, C_ROUTE), 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- P1: shared gate/up
template <bool XBF16>
__device__ void dec_shgu_item(const Layer &L, const Work &W, const void *__restrict__ x, int item) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int E = L.n_embd, F = L.n_ff, k = L.top_k;
    const int nch = E >> 3;  // 16-byte chunks per row
    const int f = item * DEC_WAVES + wave;
    if (f < F) {
        uint4 wg[8], wu[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int ch = lane + 64 * c;
            if (ch < nch) {
                wg[c] = *reinterpret_cast<const uint4 *>(L.sh_gate + (int64_t)f * E + ch * 8);
                wu[c] = *reinterpret_cast<const uint4 *>(L.sh_up + (int64_t)f * E + ch * 8);
            } else {
                wg[c] = wu[c] = make_uint4(0, 0, 0, 0);
            }
        }
        float g = 0.0f, u = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int ch = lane + 64 * c;
            if (ch < nch) {
                if (XBF16) {
                    const uint4 xv = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(x) + ch * 8);
                    g = dec_dot2(wg[c].x, xv.x, g), g = dec_dot2(wg[c].y, xv.y, g);
                    g = dec_dot2(wg[c].z, xv.z, g), g = dec_dot2(wg[c].w, xv.w, g);
                    u = dec_dot2(wu[c].x, xv.x, u), u = dec_dot2(wu[c].y, xv.y, u);
                    u = dec_dot2(wu[c].z, xv.z, u), u = dec_dot2(wu[c].w, xv.w, u);
                } else {
                    const float4 *xp = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(x) + ch * 8);
                    const float4 a = xp[0], b = xp[1];
                    const float xf[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                    const uint32_t gw[4] = {wg[c].x, wg[c].y, wg[c].z, wg[c].w};
                    const uint32_t uw[4] = {wu[c].x, wu[c].y, wu[c].z, wu[c].w};
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
        if (lane == 0) st_shared(W.hbuf + (int64_t)k * F + f, dec_silu(g) * u);
    }
    publish_item(ctr(W, C_SHGU));
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

// 64 IQ2 weights of one lane (two canonical sub-blocks) against x, before d/64
// and before the lane's x scale.  TL / TS: the level-byte and sign-byte tables
// (entry e, replica r at e * IQ2B_REPL + r).
template <bool XBF16>
__device__ __forceinline__ float dec_iq2_dot(const uint2 *TL, const uint2 *TS, uint4 q, const DecX<XBF16> &xc,
                                             int rep) {
    float acc = 0.0f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
        const uint32_t ib = sb ? q.z : q.x;   // 4 codebook indices
        const uint32_t sw = sb ? q.w : q.y;   // signs (7 x 4) | ls << 28
        uint2 lv[4], sv[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            lv[g] = TL[((ib >> (8 * g)) & 0xFFu) * IQ2B_REPL + rep];
            sv[g] = TS[((sw >> (7 * g)) & 0x7Fu) * IQ2B_REPL + rep];
        }
        float s = 0.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g)
            s = xc.dot8(iq2_expand_f16(make_uint2(lv[g].x ^ sv[g].x, lv[g].y ^ sv[g].y)), 4 * sb + g, s);
        acc = fmaf((float)(2u * (sw >> 28) + 1u), s, acc);
    }
    return acc;
}

// Wait until every router half is counted, then route locally.  Returns
// false if the bounded wait expired.
__device__ __forceinline__ bool dec_route_wait(const Layer &L, const Work &W, const DecPlan &P, RouteCache *rc,
                                               int *lds_flag) {
    if (!wait_items(W, ctr(W, C_ROUTE), (P.ep + 1) * (unsigned long long)P.n_route, lds_flag)) return false;
    if (threadIdx.x < 64) dec_topk_local(L, W, W.rhalf, rc, blockIdx.x == 0);
    __syncthreads();
    return true;
}

// Load at a 32-bit byte offset from a workgroup-uniform base.  Every plane
// read this way is below 4 GiB (the largest, an expert matrix plane, holds at
// most 256 x 4096 x 4096 / 4 bytes), and a zero-extended 32-bit offset lets
// the compiler keep the base in scalar registers and one offset per lane.
template <class T>
__device__ __forceinline__ T ld_at(const void *base, uint32_t off) {
    return *reinterpret_cast<const T *>(reinterpret_cast<const uint8_t *>(base) + off);
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
    const int e = rc->idx[j];
#pragma unroll
    for (int r = 0; r < DEC_GU_NR; ++r) {
        // rows past n_ff (if any) read row n_ff - 1; the computation drops them
        const int f = f0 + r * rpw;
        const uint32_t rb = ((uint32_t)e * F + min(f, F - 1)) * L.nbe;
        w.qg[r] = ld_at<uint4>(L.iq2_qs[0], rb * 64u + c * 16u);
        w.qu[r] = ld_at<uint4>(L.iq2_qs[1], rb * 64u + c * 16u);
        w.dg[r] = ld_at<uint16_t>(L.iq2_d[0], 2u * (rb + (c >> 2)));
        w.du[r] = ld_at<uint16_t>(L.iq2_d[1], 2u * (rb + (c >> 2)));
    }
}

template <bool XBF16>
__device__ __forceinline__ void dec_rgu_compute(const Layer &L, const Work &W, const DecX<XBF16> &xc, const uint2 *TL,
                                                const uint2 *TS, int item, const DecPlan &P, const RguW &w) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int E = L.n_embd, F = L.n_ff;
    const int lpr = E >> 6, rpw = 64 / lpr;
    const int c = lane & (lpr - 1);
    const int j = item / P.rgu_per_slot, tile = item - j * P.rgu_per_slot;
    const int f0 = (tile * DEC_WAVES + wave) * (DEC_GU_NR * rpw) + lane / lpr;
    const int rep = lane & (IQ2B_REPL - 1);
#pragma unroll
    for (int r = 0; r < DEC_GU_NR; ++r) {
        const int f = f0 + r * rpw;
        float g = dec_iq2_dot<XBF16>(TL, TS, w.qg[r], xc, rep) * (half_to_f32((uint16_t)w.dg[r]) * xc.scale);
        float u = dec_iq2_dot<XBF16>(TL, TS, w.qu[r], xc, rep) * (half_to_f32((uint16_t)w.du[r]) * xc.scale);
        g = dec_group_sum(g, lpr) * 0.015625f;
        u = dec_group_sum(u, lpr) * 0.015625f;
        if (c == 0 && f < F) st_shared(W.hbuf + (int64_t)j * F + f, dec_silu(g) * u);
    }
    publish_item(ctr(W, C_GU + j));
}

// ---------------------------------------------------------------- P3: shared down
// CPR = 16-byte chunks per lane per row (F / 512, at least 1); 16 chunk loads in
// flight per wave, i.e. 16 / CPR rows per wave.
template <int CPR>
__device__ void dec_shdn_item(const Layer &L, const Work &W, float *__restrict__ out, int item, const DecPlan &P,
                              int *lds_flag) {
    constexpr int RPW = 16 / CPR;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int E = L.n_embd, F = L.n_ff, k = L.top_k;
    const int nch = F >> 3;
    const int r0 = (item * DEC_WAVES + wave) * RPW;
    // the weights do not depend on the gate/up phase: issue them first
    uint4 wv[RPW][CPR];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
        for (int c = 0; c < CPR; ++c) {
            const int row = r0 + rr, ch = lane + 64 * c;
            wv[rr][c] = (row < E && ch < nch) ? *reinterpret_cast<const uint4 *>(L.sh_down + (int64_t)row * F + ch * 8)
                                              : make_uint4(0, 0, 0, 0);
        }
    if (!wait_items(W, ctr(W, C_SHGU), (P.ep + 1) * (unsigned long long)P.n_shgu, lds_flag)) return;
    const float *hs = W.hbuf + (int64_t)k * F;
    float hv[CPR][8];
#pragma unroll
    for (int c = 0; c < CPR; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nch) {
            // plain loads: these lines are first touched now, after every producer finished
            const float4 *p = reinterpret_cast<const float4 *>(hs + ch * 8);
            const float4 a = p[0], b = p[1];
            hv[c][0] = a.x, hv[c][1] = a.y, hv[c][2] = a.z, hv[c][3] = a.w;
            hv[c][4] = b.x, hv[c][5] = b.y, hv[c][6] = b.z, hv[c][7] = b.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) hv[c][i] = 0.0f;
        }
    }
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
        float y = 0.0f;
#pragma unroll
        for (int c = 0; c < CPR; ++c) {
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
__device__ __forceinline__ float dec_q2k_dot(uint4 qs, uint32_t sc, uint32_t dd, const float *hv, const float *hsum) {
    const uint32_t Q[4] = {qs.x, qs.y, qs.z, qs.w};
    float A = 0.0f, B = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        float dot = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t tq = (Q[s] >> (2 * u)) & 0x03030303u;
#pragma unroll
            for (int b = 0; b < 4; ++b) dot = fmaf((float)((tq >> (8 * b)) & 0xFFu), hv[16 * s + 4 * b + u], dot);
        }
        const uint32_t scb = (sc >> (8 * s)) & 0xFFu;
        A = fmaf((float)(scb & 15u), dot, A);
        B = fmaf((float)(scb >> 4), hsum[s], B);
    }
    return half_to_f32((uint16_t)(dd & 0xFFFFu)) * A - half_to_f32((uint16_t)(dd >> 16)) * B;
}

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
    const int e = rc->idx[j];
#pragma unroll
    for (int r = 0; r < DEC_DN_NR; ++r) {
        // rows past n_embd (if any) read row n_embd - 1; the computation drops them
        const int row = r0 + r * rpw;
        const uint32_t rb = ((uint32_t)e * E + min(row, E - 1)) * L.nbf;
        w.qs[r] = ld_at<uint4>(L.q2k_qs, rb * 64u + c * 16u);
        w.sc[r] = ld_at<uint32_t>(L.q2k_sc, rb * 16u + c * 4u);
        w.dd[r] = ld_at<uint32_t>(L.q2k_dd, 4u * (rb + (c >> 2)));
    }
}

// Returns false if the wait for the slot's gate/up items expired.
__device__ __forceinline__ bool dec_rdn_compute(const Layer &L, const Work &W, float *__restrict__ out, int item,
                                                const DecPlan &P, int *lds_flag, const RouteCache *rc, const RdnW &w) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int E = L.n_embd, F = L.n_ff;
    const int lpr = F >> 6, rpw = 64 / lpr;
    const int c = lane & (lpr - 1);
    const int j = item / P.rdn_per_slot, tile = item - j * P.rdn_per_slot;
    const int r0 = (tile * DEC_WAVES + wave) * (DEC_DN_NR * rpw) + lane / lpr;
    const float wgt = rc->w[j];
    if (!wait_items(W, ctr(W, C_GU + j), (P.ep + 1) * (unsigned long long)P.rgu_per_slot, lds_flag)) return false;
    float hv[64], hsum[4];
    // plain loads: these lines are first touched now, after every producer finished
    const float4 *hp = reinterpret_cast<const float4 *>(W.hbuf + (int64_t)j * F + 64 * c);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float4 v = hp[i];
        hv[4 * i] = v.x, hv[4 * i + 1] = v.y, hv[4 * i + 2] = v.z, hv[4 * i + 3] = v.w;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) a += hv[16 * s + i];
        hsum[s] = a;
    }
#pragma unroll
    for (int r = 0; r < DEC_DN_NR; ++r) {
        const int row = r0 + r * rpw;
        float y = dec_q2k_dot(w.qs[r], w.sc[r], w.dd[r], hv, hsum);
        y = dec_group_sum(y, lpr);
        if (c == 0 && row < E) atomicAdd(out + row, wgt * y);
    }
    return true;
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
    const int G = gridDim.x;
    // item order: router, shared gate/up, routed gate/up, routed down, shared down;
    // every wait is on an earlier phase
    const int b0 = P.n_route, b1 = b0 + P.n_shgu, b2 = b1 + P.n_rgu, b3 = b2 + P.n_rdn;
    // one loop per phase (the same items in the same order as a single loop
    // over all of them), so that each phase's registers are allocated on their own
    // loads that depend on nothing are issued before the router item: this
    // thread's codebook entry and the lane's slice of x for the routed gate/up
    // (lane c of a routed gate/up row holds x[64 c .. 64 c + 63])
    const uint32_t cb = L.codebook[threadIdx.x & 255];
    DecX<XBF16> xc;
    xc.load(x, 64 * ((threadIdx.x & 63) & ((L.n_embd >> 6) - 1)));
    int it = blockIdx.x;
    for (; it < b0; it += G) dec_route_item<XBF16>(L, W, x, it, &lds_flag, lds_part, P);
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
    // the shared expert's gate/up needs no routing: it streams while the
    // router halves are counted
    for (; it < b1; it += G) dec_shgu_item<XBF16>(L, W, x, it - b0);
    bool ok = dec_route_wait(L, W, P, &rc, &lds_flag);
    // routed gate/up: the next item's weights are in flight while this one is computed
    if (ok && it < b2) {
        RguW wa, wb;   // two named buffers, alternating (no copies)
        dec_rgu_load(L, P, &rc, it - b1, wa);
        for (;;) {
            bool more = it + G < b2;
            if (more) dec_rgu_load(L, P, &rc, it + G - b1, wb);
            dec_rgu_compute<XBF16>(L, W, xc, TL, TS, it - b1, P, wa);
            it += G;
            if (!more) break;
            more = it + G < b2;
            if (more) dec_rgu_load(L, P, &rc, it + G - b1, wa);
            dec_rgu_compute<XBF16>(L, W, xc, TL, TS, it - b1, P, wb);
            it += G;
            if (!more) break;
        }
    }
    // routed down: the same pipelining; weights do not wait for the gate/up phase
    if (ok && it < b3) {
        RdnW wa, wb;
        dec_rdn_load(L, P, &rc, it - b2, wa);
        for (;;) {
            bool more = it + G < b3;
            if (more) dec_rdn_load(L, P, &rc, it + G - b2, wb);
            if (!dec_rdn_compute(L, W, out, it - b2, P, &lds_flag, &rc, wa)) { ok = false; break; }
            it += G;
            if (!more) break;
            more = it + G < b3;
            if (more) dec_rdn_load(L, P, &rc, it + G - b2, wa);
            if (!dec_rdn_compute(L, W, out, it - b2, P, &lds_flag, &rc, wb)) { ok = false; break; }
            it += G;
            if (!more) break;
        }
    }
    for (; ok && it < P.total; it += G) {
        switch (P.shdn_cpr) {
            case 1: dec_shdn_item<1>(L, W, out, it - b3, P, &lds_flag); break;
            case 2: dec_shdn_item<2>(L, W, out, it - b3, P, &lds_flag); break;
            case 4: dec_shdn_item<4>(L, W, out, it - b3, P, &lds_flag); break;
            default: dec_shdn_item<8>(L, W, out, it - b3, P, &lds_flag); break;
        }
    }
    // a bounded wait expired somewhere: make the failure visible in the output
    if (blockIdx.x == 0 && threadIdx.x == 0 &&
        __hip_atomic_load(ctr(W, C_ERR), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
        out[0] = __builtin_nanf("");
}

static DecPlan make_plan(const Layer &L) {
    DecPlan P{};
    const int E = L.n_embd, F = L.n_ff, k = L.top_k;
    P.n_route = 2 * L.n_expert;  // half an expert row per item
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
                               unsigned long long ep, hipStream_t s) {
    DecPlan P = make_plan(L);
    P.ep = ep;
    Layer Lc = L;
    Work Wc = W;
    const void *xc = x;
    float *oc = out;
    void *args[] = {&Lc, &Wc, &xc, &oc, &P};
    const void *fn = (L.act_dtype == 1) ? reinterpret_cast<const void *>(&k_decode_fused<true>)
                                        : reinterpret_cast<const void *>(&k_decode_fused<false>);
    hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(DEC_THREADS), args, 0, s);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace ds4
