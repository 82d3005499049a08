// small.hip - the MoE block for small batches (2..SMALL_MAX_TOK tokens, bf16
// activations) in two persistent launches after the router.
//
// Speculative decoding verifies k + 1 tokens per step ("ds4 深度实战...",
// sections 4.2 and 4.4), and such small batches are bound by memory like
// decode (same page, section 5.1): each selected expert's weights should
// stream from HBM once per call, for all of the tokens that chose it, with
// every CU streaming.  Here:
//   k_small_gateup: every workgroup stages all tokens' x in LDS (fp16 under a
//     per-token power-of-two scale), the IQ2 level table and the sign-mask
//     table (mfma_ops.h), then streams a
//     contiguous range of units: the shared expert's gate and up (16 rows x
//     256 K, bf16) and each selected expert's gate and up (16 rows x up to
//     eight 256-K blocks, IQ2).  A unit is one wave's MFMA tile: 16 weight
//     rows against all of the unit's tokens.  Its partial sums are added into
//     an fp32 buffer (row t k + j for slot j of token t, row SMALL_MAX_TOK k +
//     t for the shared expert of token t).
//   k_small_down: every workgroup stages the h = SiLU(g) u vectors its units
//     need from those sums (fp16, per-vector power-of-two scale), then
//     streams its units: each selected expert's down rows (16 rows x n_ff,
//     Q2_K) and the shared down rows (16 rows x 256 K, bf16), adding w y into
//     the residual.  It also clears the other sum buffer, which the next call
//     will use: the two buffers alternate, so no buffer is cleared while it
//     is read.
// Units are split over the workgroups in contiguous ranges and dealt
// round-robin to each workgroup's 12 waves; a wave computes each half of a
// unit while the next half's weights are in flight (two register buffers,
// three waves per SIMD: measured faster than 8 waves with a ring of four
// buffers, and than 16 waves with one).  A lane loads a quarter of a row block
// (IQ2, Q2_K) or 16 bytes of a row part (bf16), so one load instruction reads
// each 128-byte line only in part and the next few read the rest: weights
// are read with ordinary loads, which keep the line in L2 for them (a
// non-temporal load would let every part fetch the line again).
//
// Numerics are the grouped GEMMs': the routed weights enter the MFMAs rounded
// to fp16 (mfma_ops.h), the shared expert's bf16 weights are converted to
// fp16 (exact in fp16's normal range), and x and h are fp16 under power-of-two
// scales (no overflow; values below 2^-28 of the vector's largest lose bits),
// accumulated in fp32.
#include "common.h"
#include "iq2_tables.h"
#include "mfma_ops.h"

namespace ds4 {

constexpr int SB_WAVES = 12;                        // one workgroup per CU, 3 waves per SIMD
constexpr int SB_THREADS = 64 * SB_WAVES;
constexpr int SB_XV = (SMALL_MAX_TOK * 4096 / 8 + SB_THREADS - 1) / SB_THREADS;  // x vectors (16 B) per thread at most
constexpr int SB_HV = (SMALL_MAX_TOK * SMALL_MAX_FF / 8 + SB_THREADS - 1) / SB_THREADS;  // h groups of 8 per thread at most
static_assert(SB_THREADS % 32 == 0, "a group of 32 lanes covers 32 consecutive vectors");
constexpr int SB_SLOTS = SMALL_MAX_TOK * MAX_TOPK;  // (token, expert) selections at most
constexpr int SB_XP = 2 * 4096 + 16;                // x row pitch in LDS, bytes (n_embd <= 4096; 16 B * odd)
constexpr int SB_HP = 2 * SMALL_MAX_FF + 16;        // routed h row pitch, bytes
constexpr int SB_SHK = 512;                         // shared down: K values of h staged (two 256-K parts)
constexpr int SB_SP = 2 * SB_SHK + 16;              // shared h row pitch, bytes

// The call's routing, built from the selections the router kernel wrote
// earlier on the stream (W.idx, W.w: expert and weight of selection q = t k +
// j): active expert u = e[u] (ascending), in weight slot wslot[u], with cnt[u]
// selections at list positions beg[u].. (entries q, ascending t); wq[q] is
// selection q's renormalised weight.
struct SbRoute {
    int U;
    int e[SB_SLOTS], wslot[SB_SLOTS], beg[SB_SLOTS], cnt[SB_SLOTS];
    int lst[SB_SLOTS], sel[SB_SLOTS];
    float wq[SB_SLOTS];
    int wtot[4], wact[4];
};

// Every workgroup builds the same tables (a count per expert, a scan over the
// experts, each selection's rank among the earlier ones of its expert);
// with export_lists, it also writes the per-expert lists to W (offsets,
// active experts, entries) as the router's own list step would, for the
// routing export.  cnt: MAX_EXPERT + 1 ints of LDS.
__device__ void sb_read_route(const Layer &L, const Work &W, int n, SbRoute &R, int *cnt, bool export_lists) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int NE = L.n_expert, nq = n * L.top_k;
    int e = 0;
    if (tid < nq) {
        e = W.idx[tid];
        R.sel[tid] = e;
        R.wq[tid] = W.w[tid];
    }
    if (tid <= MAX_EXPERT) cnt[tid] = 0;
    __syncthreads();
    if (tid < nq) atomicAdd(&cnt[e], 1);
    __syncthreads();
    // thread x < 256 holds expert x: exclusive scans of the counts and of the
    // active flags, by wave scans and the four wave totals
    const int c = tid < NE ? cnt[tid] : 0;
    int v = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    const uint64_t am = __ballot(c > 0);
    if (tid < 256 && lane == 63) R.wtot[wave] = v;
    if (tid < 256 && lane == 0) R.wact[wave] = __popcll(am);
    __syncthreads();
    if (tid < 256) {
        int pre = 0, apre = 0;
        for (int w = 0; w < wave; ++w) pre += R.wtot[w], apre += R.wact[w];
        const int start = pre + v - c;
        if (c > 0) {
            const int u = apre + __popcll(am & ((1ull << lane) - 1ull));
            R.e[u] = tid;
            R.wslot[u] = expert_slot(L, tid);
            R.beg[u] = start;
            R.cnt[u] = c;
            if (export_lists) W.active[1 + u] = tid;
        }
        if (export_lists && tid <= NE) W.offsets[tid] = start;  // (tid == NE: start = nq)
        if (tid == 255) {
            R.U = apre + __popcll(am);
            if (export_lists) W.active[0] = R.U;
        }
        cnt[tid] = start;  // offsets, for the entries below (read after the barrier)
    }
    if (export_lists && NE == 256 && tid == 256) W.offsets[256] = nq;
    __syncthreads();
    if (wave == 0) {
        // entry position: the expert's offset plus the earlier selections of
        // it, counted by a wave match (every selection is in wave 0: nq <= 64)
        static_assert(SB_SLOTS <= 64 && MAX_EXPERT <= 256, "the selections fit one wave, experts 8 bits");
        const bool v = tid < nq;
        const uint64_t m = wave_match_any((uint32_t)e, 8) & __ballot(v);
        if (v) {
            const int r = __popcll(m & ((1ull << lane) - 1ull));
            R.lst[cnt[e] + r] = tid;
            if (export_lists) W.list[cnt[e] + r] = tid;
        }
    }
    __syncthreads();
}

// 8 bf16 weights -> fp16 (exact for magnitudes in [2^-14, 65504])
__device__ __forceinline__ half8 sb_bf16_to_half8(const uint4 &w) {
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
    half8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[2 * i] = (_Float16)__uint_as_float(a[i] << 16);
        r[2 * i + 1] = (_Float16)__uint_as_float(a[i] & 0xFFFF0000u);
    }
    return r;
}

// Power-of-two scale exponent putting a vector's largest magnitude mx in
// [2^14, 2^15) (clamped for zero or extreme vectors).
__device__ __forceinline__ int sb_scale_exp(float mx) {
    const int ex = (int)((__float_as_uint(mx) >> 23) & 0xFFu) - 127;
    return min(max(ex - 14, -100), 100);
}
__device__ __forceinline__ float sb_pow2(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }

// Load at a byte offset from a base.
template <class T>
__device__ __forceinline__ T ld_at(const void *base, int off) {
    return *reinterpret_cast<const T *>(reinterpret_cast<const uint8_t *>(base) + off);
}

// Units are split over the workgroups by estimated cost: a routed unit (8
// IQ2 / Q2_K blocks, 64 MFMA steps with table lookups) costs more than a
// shared one (8 steps of bf16), in the ratio measured per unit.  The units of
// workgroup b are those whose start cost lies in [C b / G, C (b + 1) / G);
// unit u of a list of na units of cost ca then nb units of cost cb starts at
// u ca (u < na) or na ca + (u - na) cb.
constexpr int SB_GU_COST_SHARED = 4, SB_GU_COST_ROUTED = 9;
constexpr int SB_DN_COST_ROUTED = 3, SB_DN_COST_SHARED = 1;
// Units (of the list above) that start below cost c.
__device__ __forceinline__ int sb_units_below(int64_t c, int na, int ca, int nb, int cb) {
    const int64_t ea = (int64_t)na * ca;
    if (c <= ea) return (int)((c + ca - 1) / ca);
    return na + (int)min<int64_t>((c - ea + cb - 1) / cb, nb);
}
__device__ __forceinline__ void sb_range(int na, int ca, int nb, int cb, int &g0, int &g1) {
    const int64_t C = (int64_t)na * ca + (int64_t)nb * cb;
    g0 = sb_units_below(C * blockIdx.x / gridDim.x, na, ca, nb, cb);
    g1 = sb_units_below(C * (blockIdx.x + 1) / gridDim.x, na, ca, nb, cb);
}

// Maximum of a non-negative value over each group of 32 consecutive lanes,
// in the group's last lane (lane 31 or 63), by DPP row shifts and one row
// broadcast: plain VALU work (no round trip through LDS).  All lanes active.
__device__ __forceinline__ float sb_max32_last(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, true)));  // row_shr:1
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, true)));  // row_shr:2
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, true)));  // row_shr:4
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, true)));  // row_shr:8
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false))); // row_bcast:15
    return v;
}

// ---------------------------------------------------------------- gate/up
// 16-bit element j (0..7) of a 16-byte group.
__device__ __forceinline__ uint32_t sb_u16_of(const uint4 &v, int j) {
    const uint32_t w = j < 2 ? v.x : j < 4 ? v.y : j < 6 ? v.z : v.w;
    return (w >> (16 * (j & 1))) & 0xFFFFu;
}
// 32-bit element j (0..7) of two 16-byte groups.
__device__ __forceinline__ uint32_t sb_u32_of(const uint4 &a, const uint4 &b, int j) {
    const uint4 v = j < 4 ? a : b;
    const int i = j & 3;
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Half h of a unit's weights for this lane: 4 gate uint4 (q[0..3]) and 4 up
// uint4 (q[4..7]) -- a routed unit's blocks 4 h .. 4 h + 3, a shared unit's
// steps 4 h .. 4 h + 3 -- and the gate and up block scales d of the row's
// 16-byte group holding the unit's blocks (element doff + s for block s;
// routed units only, shared units load valid unused words there).  A wave
// computes one half while the next one's loads are in flight.
struct SbW {
    uint4 q[8];
    uint4 dg, du;
    int doff;
};

// Unit i: i < ns shared (tile i / nbe, 256-K part i % nbe; lane group g of
// step s holds K 32 s + 8 g of the part, so a load reads 64 contiguous bytes
// of each row); else routed (slot u, tile, part of bpu blocks).  Every load
// is issued whatever the unit (addresses are selected, loads are never
// skipped), so the compiler's waits count the same loads on every path; with
// `none` every address is the same 16 bytes of the codebook (a cache hit, the
// values unused).
__device__ __forceinline__ void sb_gu_load(const Layer &L, const SbRoute &R, int i, int h, int ns, int TG, int pr,
                                           int bpu, bool none, SbW &w) {
    const int lane = threadIdx.x & 63, rl = lane & 15, grp = lane >> 4;
    const int E = L.n_embd, F = L.n_ff, nbe = L.nbe;
    const bool sh = i < ns;
    const uint8_t *q0, *q1, *d0, *d1;
    int qs, last;
    w.doff = 0;
    if (sh) {
        const int tile = i / nbe, part = i - tile * nbe;
        const int64_t o = ((int64_t)(16 * tile + rl) * E + 256 * part + 8 * grp) * 2;
        q0 = reinterpret_cast<const uint8_t *>(L.sh_gate) + o;
        q1 = reinterpret_cast<const uint8_t *>(L.sh_up) + o;
        d0 = d1 = reinterpret_cast<const uint8_t *>(L.iq2_d[0]);
        qs = 64, last = 7;
    } else {
        const int r = i - ns, per = TG * pr;
        // (past the last unit, with `none` set, u may reach U: clamped, the address is not used)
        const int u = min(r / per, R.U - 1), rem = r - u * per, tile = rem / pr, part = rem - tile * pr;
        const int64_t rb = ((int64_t)R.wslot[u] * F + 16 * tile + rl) * nbe + part * bpu;
        q0 = L.iq2_qs[0] + rb * 64 + 16 * grp;
        q1 = L.iq2_qs[1] + rb * 64 + 16 * grp;
        // the unit's bpu scales lie in one 16-byte group (bpu = 8 at rb = 0 mod
        // 8, or a row's whole nbe < 8 blocks)
        d0 = reinterpret_cast<const uint8_t *>(L.iq2_d[0] + (rb & ~(int64_t)7));
        d1 = reinterpret_cast<const uint8_t *>(L.iq2_d[1] + (rb & ~(int64_t)7));
        w.doff = (int)(rb & 7);
        qs = 64, last = bpu - 1;
    }
    if (none) {
        q0 = q1 = d0 = d1 = reinterpret_cast<const uint8_t *>(L.codebook);
        qs = 0;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int ss = min(4 * h + s, last);
        w.q[s] = ld_at<uint4>(q0, ss * qs);
        w.q[4 + s] = ld_at<uint4>(q1, ss * qs);
    }
    w.dg = ld_at<uint4>(d0, 0);
    w.du = ld_at<uint4>(d1, 0);
}

// Half h of unit i into the gate and up accumulators (16 tokens x 16 rows).
// Lanes past the unit's tokens read its first token's x: their products land
// in C rows never stored.
__device__ __forceinline__ void sb_gu_compute(const Layer &L, const SbRoute &R, const uint4 *T, const uint4 *ST,
                                              const uint8_t *xs,
                                              int i, int h, int ns, int TG, int pr, int bpu, int n, const SbW &w,
                                              floatx4 &ag, floatx4 &au) {
    const int lane = threadIdx.x & 63, rl = lane & 15, grp = lane >> 4;
    const int k = L.top_k, nbe = L.nbe;
    if (i < ns) {
        const int tile = i / nbe, part = i - tile * nbe;
        const uint8_t *xr = xs + (rl < n ? rl : 0) * SB_XP + 2 * (256 * part + 8 * grp) + 256 * h;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const half8 a = *reinterpret_cast<const half8 *>(xr + 64 * s);
            ag = mfma_f16(a, sb_bf16_to_half8(w.q[s]), ag);
            au = mfma_f16(a, sb_bf16_to_half8(w.q[4 + s]), au);
        }
        return;
    }
    const int r = i - ns, per = TG * pr;
    const int u = r / per, part = (r - u * per) % pr;
    const int beg = R.beg[u], cnt = R.cnt[u];
    const int tq = R.lst[beg + (rl < cnt ? rl : 0)] / k;
    const uint8_t *xr = xs + tq * SB_XP + 2 * (256 * part * bpu + 64 * grp);
    half2v sg, su;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int b = 4 * h + s;  // block of the unit
        if (b >= bpu) break;
        const uint32_t dgb = sb_u16_of(w.dg, w.doff + b), dub = sb_u16_of(w.du, w.doff + b);
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
            const uint4 lg = iq2_b_lookup(T, w.q[s], cc, rl), lu = iq2_b_lookup(T, w.q[4 + s], cc, rl);
            const uint4 mg = iq2_s_lookup(ST, w.q[s], cc, rl), mu = iq2_s_lookup(ST, w.q[4 + s], cc, rl);
            const half8 a = *reinterpret_cast<const half8 *>(xr + 512 * b + 16 * cc);
            const half8 bg = iq2_b_finish_masked(lg, mg, w.q[s], (uint16_t)dgb, cc, sg);
            const half8 bu = iq2_b_finish_masked(lu, mu, w.q[4 + s], (uint16_t)dub, cc, su);
            ag = mfma_f16(a, bg, ag);
            au = mfma_f16(a, bu, au);
        }
    }
}

// Unit i's sums, times the x scales, added into the buffer.
__device__ __forceinline__ void sb_gu_store(const Layer &L, const SbRoute &R, const float *xsc, int i, int ns,
                                            int TG, int pr, int n, const floatx4 &ag, const floatx4 &au,
                                            float *__restrict__ gu) {
    const int lane = threadIdx.x & 63, rl = lane & 15, grp = lane >> 4;
    const int F = L.n_ff, k = L.top_k, nbe = L.nbe;
    if (i < ns) {
        const int f = 16 * (i / nbe) + rl;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int t = 4 * grp + v;
            if (t < n) {
                float *row = gu + (int64_t)(SMALL_MAX_TOK * k + t) * 2 * F + f;
                atomicAdd(row, ag[v] * xsc[t]);
                atomicAdd(row + F, au[v] * xsc[t]);
            }
        }
        return;
    }
    const int r = i - ns, per = TG * pr;
    const int u = r / per, f = 16 * ((r - u * per) / pr) + rl;
    const int beg = R.beg[u], cnt = R.cnt[u];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int ii = 4 * grp + v;
        if (ii < cnt) {
            const int q = R.lst[beg + ii];
            const float sc = xsc[q / k];
            float *row = gu + (int64_t)q * 2 * F + f;
            atomicAdd(row, ag[v] * sc);
            atomicAdd(row + F, au[v] * sc);
        }
    }
}

// grid: one workgroup per CU (LDS: the level and sign tables and x), SB_THREADS threads.
__global__ __launch_bounds__(SB_THREADS, 1) void k_small_gateup(Layer L, Work W, const uint16_t *__restrict__ x,
                                                                int n, float *__restrict__ gu) {
    __shared__ uint4 T[256 * IQ2_REPL];
    __shared__ uint4 ST[128 * IQ2S_REPL];
    __shared__ __align__(16) uint8_t xs[SMALL_MAX_TOK * SB_XP];
    __shared__ SbRoute R;
    __shared__ int ecnt[MAX_EXPERT + 1];
    __shared__ uint32_t xmax[SMALL_MAX_TOK];
    __shared__ float xsc[SMALL_MAX_TOK];
    const int tid = threadIdx.x, wave = tid >> 6;
    const int E = L.n_embd, F = L.n_ff, nbe = L.nbe;
    const int e8 = E >> 3, nv = n * e8;  // 16-byte vectors of x per token, in all
    // x and the codebook first (the thread's vectors tid + SB_THREADS j of x:
    // n E / 8 <= SB_XV SB_THREADS)
    const uint32_t cbw = tid < 256 ? L.codebook[tid] : 0u;
    uint4 xr[SB_XV];
#pragma unroll
    for (int j = 0; j < SB_XV; ++j) {
        const int i = min(tid + SB_THREADS * j, nv - 1);
        xr[j] = *reinterpret_cast<const uint4 *>(x + 8 * (int64_t)i);
    }
    if (tid < SMALL_MAX_TOK) xmax[tid] = 0u;
    sb_read_route(L, W, n, R, ecnt, blockIdx.x == 0);
    // units: shared (F / 16 tiles x nbe parts), then routed (U slots x tiles x parts)
    const int TG = F >> 4, bpu = min(8, nbe), pr = nbe / bpu;
    const int ns = L.n_shared ? TG * nbe : 0;
    int g0, g1;
    sb_range(ns, SB_GU_COST_SHARED, R.U * TG * pr, SB_GU_COST_ROUTED, g0, g1);
    int i = g0 + wave;
    // the first half unit's weights stream while x and the table are staged
    SbW wa, wb;
    sb_gu_load(L, R, i, 0, ns, TG, pr, bpu, i >= g1, wa);
    // per-token maxima of |x| (32 consecutive vectors always belong to one token)
#pragma unroll
    for (int j = 0; j < SB_XV; ++j) {
        const int iv = tid + SB_THREADS * j;
        if (SB_THREADS * j >= nv) break;
        const uint32_t a[4] = {xr[j].x, xr[j].y, xr[j].z, xr[j].w};
        float m = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) m = fmaxf(m, fmaxf(fabsf(bf16_to_f32((uint16_t)(a[q] & 0xFFFFu))),
                                                      fabsf(bf16_to_f32((uint16_t)(a[q] >> 16)))));
        m = sb_max32_last(m);
        if (iv < nv && (tid & 31) == 31) atomicMax(&xmax[iv / e8], __float_as_uint(m));
    }
    if (tid < 256) iq2_lut_entry<true>(T, tid, cbw);
    iq2_build_sign_table(ST, tid, SB_THREADS);
    __syncthreads();
    if (tid < n) xsc[tid] = sb_pow2(sb_scale_exp(__uint_as_float(xmax[tid])));
#pragma unroll
    for (int j = 0; j < SB_XV; ++j) {
        const int iv = tid + SB_THREADS * j;
        if (SB_THREADS * j >= nv) break;
        if (iv < nv) {
            const int t = iv / e8;
            const float down = sb_pow2(-sb_scale_exp(__uint_as_float(xmax[t])));
            const uint32_t a[4] = {xr[j].x, xr[j].y, xr[j].z, xr[j].w};
            half8 h;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                h[2 * q] = (_Float16)(bf16_to_f32((uint16_t)(a[q] & 0xFFFFu)) * down);
                h[2 * q + 1] = (_Float16)(bf16_to_f32((uint16_t)(a[q] >> 16)) * down);
            }
            *reinterpret_cast<half8 *>(xs + t * SB_XP + 16 * (iv - t * e8)) = h;
        }
    }
    __syncthreads();
    // the wave's units i, i + SB_WAVES, .., by halves in two named buffers:
    // each half is computed while the next one's loads are in flight
    for (; i < g1; i += SB_WAVES) {
        sb_gu_load(L, R, i, 1, ns, TG, pr, bpu, false, wb);
        floatx4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
        sb_gu_compute(L, R, T, ST, xs, i, 0, ns, TG, pr, bpu, n, wa, ag, au);
        const int nx = i + SB_WAVES;
        sb_gu_load(L, R, nx, 0, ns, TG, pr, bpu, nx >= g1, wa);
        sb_gu_compute(L, R, T, ST, xs, i, 1, ns, TG, pr, bpu, n, wb, ag, au);
        sb_gu_store(L, R, xsc, i, ns, TG, pr, n, ag, au, gu);
    }
}

// ---------------------------------------------------------------- down
// Half h of a unit's weights for this lane: routed, per 256-K block b = 4 h
// .. 4 h + 3 (nbf <= 8) the lane's 16 qs bytes and 4 scale bytes, and the
// row's words d | dmin; shared, per step 4 h .. 4 h + 3 the 8 bf16 weights
// (scales: valid unused words).
struct SbDW {
    uint4 q[4];
    uint32_t sc[4];
    uint4 dd0, dd1;  // d | dmin of the row's blocks: element doff + b of the two 16-byte groups
    int doff;
};

// Unit i: i < nr routed (slot i / TE, tile i % TE: 16 rows of n_embd, all of
// n_ff); else shared, 256-K part major (part j / TE, tile j % TE, j = i - nr;
// K as for the shared gate/up); `none` as for sb_gu_load.
__device__ __forceinline__ void sb_dn_load(const Layer &L, const SbRoute &R, int i, int h, int nr, int TE,
                                           bool none, SbDW &w) {
    const int lane = threadIdx.x & 63, rl = lane & 15, grp = lane >> 4;
    const int E = L.n_embd, F = L.n_ff, nbf = L.nbf;
    const uint8_t *q0, *s0, *d0, *d1;
    int qs, ss, last;
    w.doff = 0;
    if (i < nr) {
        const int u = i / TE, tile = i - u * TE;
        const int64_t rb = ((int64_t)R.wslot[u] * E + 16 * tile + rl) * nbf;
        q0 = L.q2k_qs + rb * 64 + 16 * grp;
        s0 = L.q2k_sc + rb * 16 + 4 * grp;
        // the row's nbf words d | dmin: two 16-byte groups (nbf = 8 at rb = 0
        // mod 8), or one group holding all nbf <= 4 of them (read twice)
        const int64_t g0 = rb & ~(int64_t)3;
        d0 = reinterpret_cast<const uint8_t *>(L.q2k_dd + g0);
        d1 = reinterpret_cast<const uint8_t *>(L.q2k_dd + (nbf > 4 ? g0 + 4 : g0));
        w.doff = (int)(rb & 3);
        qs = 64, ss = 16, last = nbf - 1;
    } else {
        const int j = i - nr, part = j / TE, tile = j - part * TE;
        q0 = reinterpret_cast<const uint8_t *>(L.sh_down) +
             ((int64_t)(16 * tile + rl) * F + 256 * part + 8 * grp) * 2;
        s0 = d0 = d1 = reinterpret_cast<const uint8_t *>(L.q2k_dd);
        qs = 64, ss = 0, last = 7;
    }
    if (none) {
        q0 = s0 = d0 = d1 = reinterpret_cast<const uint8_t *>(L.codebook);
        qs = ss = 0;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int b = min(4 * h + s, last);
        w.q[s] = ld_at<uint4>(q0, b * qs);
        w.sc[s] = ld_at<uint32_t>(s0, b * ss);
    }
    w.dd0 = ld_at<uint4>(d0, 0);
    w.dd1 = ld_at<uint4>(d1, 0);
}

// Half h of unit i into the accumulator (16 tokens x 16 rows).
__device__ __forceinline__ void sb_dn_compute(const Layer &L, const SbRoute &R, const uint2 *QT, const uint8_t *hr,
                                              int u0, const uint8_t *hsh, int kp0, int i, int h, int nr, int TE,
                                              int n, const SbDW &w, floatx4 &acc) {
    const int lane = threadIdx.x & 63, rl = lane & 15, grp = lane >> 4;
    const int nbf = L.nbf;
    if (i >= nr) {
        const int j = i - nr, part = j / TE;
        const uint8_t *hp = hsh + (rl < n ? rl : 0) * SB_SP + 2 * (256 * (part - kp0) + 8 * grp) + 256 * h;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc = mfma_f16(*reinterpret_cast<const half8 *>(hp + 64 * s), sb_bf16_to_half8(w.q[s]), acc);
        return;
    }
    const int u = i / TE, su = u - u0, cnt = R.cnt[u];
    const uint8_t *hp = hr + (su * SMALL_MAX_TOK + (rl < cnt ? rl : 0)) * SB_HP + 2 * 64 * grp;
    half8 dsc, msc;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int b = 4 * h + s;  // block of the row
        if (b >= nbf) break;
        const uint32_t ddb = sb_u32_of(w.dd0, w.dd1, w.doff + b);
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
            const uint4 qv = q2k_b_lookup(QT, w.q[s], cc, rl);
            const half8 a = *reinterpret_cast<const half8 *>(hp + 512 * b + 16 * cc);
            acc = mfma_f16(a, q2k_b_finish(qv, w.sc[s], ddb, cc, dsc, msc), acc);
        }
    }
}

// Unit i's rows, times the routing weight and the h scales, added into out.
__device__ __forceinline__ void sb_dn_store(const Layer &L, const SbRoute &R, const float *hsc, int u0,
                                            const float *shsc, int i, int nr, int TE, int n, const floatx4 &acc,
                                            float *__restrict__ out) {
    const int lane = threadIdx.x & 63, rl = lane & 15, grp = lane >> 4;
    const int E = L.n_embd, k = L.top_k;
    if (i >= nr) {
        const int row = 16 * ((i - nr) % TE) + rl;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int t = 4 * grp + v;
            if (t < n) atomicAdd(out + (int64_t)t * E + row, acc[v] * shsc[t]);
        }
        return;
    }
    const int u = i / TE, row = 16 * (i - u * TE) + rl, su = u - u0;
    const int beg = R.beg[u], cnt = R.cnt[u];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int ii = 4 * grp + v;
        if (ii < cnt) {
            const int q = R.lst[beg + ii];
            atomicAdd(out + (int64_t)(q / k) * E + row, R.wq[q] * acc[v] * hsc[su * SMALL_MAX_TOK + ii]);
        }
    }
}

// Staging of h = SiLU(g) u for `rows` rows of sums (row r of slot u's list,
// or row SMALL_MAX_TOK k + r, the shared expert of token r, when u < 0), K
// range [k0, k0 + nk), into LDS as fp16 under a power-of-two scale per row:
// dst row r at dst + r * pitch, its scale (2^e, undoing the staging's 2^-e)
// in sc[r].  nk is a multiple of 256 and rows * nk <= SB_THREADS * 8 SB_HV.
// In two parts: sb_stage_issue loads the thread's sums (so other loads can
// be issued behind them), sb_stage_finish forms h, takes the per-row maxima
// (hmax, zero on entry) and stores.
struct SbStage {
    float4 g[SB_HV][2], u[SB_HV][2];
};
__device__ __forceinline__ void sb_stage_issue(const float *__restrict__ gu, int F, const SbRoute &R, int u, int k,
                                               int rows, int k0, int nk, SbStage &st) {
    const int tid = threadIdx.x, n8 = nk >> 3;  // groups of 8 values per row
#pragma unroll
    for (int j = 0; j < SB_HV; ++j) {
        if (SB_THREADS * j >= rows * n8) break;  // uniform
        // past the last group: the last row again (in range, unused)
        const int iv = tid + SB_THREADS * j, r = min(iv / n8, rows - 1), c = 8 * (iv - (iv / n8) * n8);
        const int src = u >= 0 ? R.lst[R.beg[u] + r] : SMALL_MAX_TOK * k + r;
        const float *p = gu + (int64_t)src * 2 * F + k0 + min(c, nk - 8);
        st.g[j][0] = *reinterpret_cast<const float4 *>(p);
        st.g[j][1] = *reinterpret_cast<const float4 *>(p + 4);
        st.u[j][0] = *reinterpret_cast<const float4 *>(p + F);
        st.u[j][1] = *reinterpret_cast<const float4 *>(p + F + 4);
    }
}
__device__ void sb_stage_finish(int rows, int nk, const SbStage &st, uint8_t *dst, int pitch, float *sc,
                                uint32_t *hmax) {
    const int tid = threadIdx.x, n8 = nk >> 3, nv = rows * n8;
    float h[SB_HV][8];
#pragma unroll
    for (int j = 0; j < SB_HV; ++j) {
        if (SB_THREADS * j >= nv) break;  // uniform, as in sb_stage_issue
        const int iv = tid + SB_THREADS * j;
        const float g[8] = {st.g[j][0].x, st.g[j][0].y, st.g[j][0].z, st.g[j][0].w,
                            st.g[j][1].x, st.g[j][1].y, st.g[j][1].z, st.g[j][1].w};
        const float u[8] = {st.u[j][0].x, st.u[j][0].y, st.u[j][0].z, st.u[j][0].w,
                            st.u[j][1].x, st.u[j][1].y, st.u[j][1].z, st.u[j][1].w};
        float m = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            h[j][q] = silu(g[q]) * u[q];
            m = fmaxf(m, fabsf(h[j][q]));
        }
        // 32 consecutive groups (256 values) always belong to one row
        m = sb_max32_last(m);
        if (iv < nv && (tid & 31) == 31) atomicMax(&hmax[iv / n8], __float_as_uint(m));
    }
    __syncthreads();
    if (tid < rows) sc[tid] = sb_pow2(sb_scale_exp(__uint_as_float(hmax[tid])));
#pragma unroll
    for (int j = 0; j < SB_HV; ++j) {
        const int iv = tid + SB_THREADS * j;
        if (SB_THREADS * j < nv && iv < nv) {
            const int r = iv / n8, c = 8 * (iv - r * n8);
            const float down = sb_pow2(-sb_scale_exp(__uint_as_float(hmax[r])));
            half8 o;
#pragma unroll
            for (int q = 0; q < 8; ++q) o[q] = (_Float16)(h[j][q] * down);
            *reinterpret_cast<half8 *>(dst + r * pitch + 2 * c) = o;
        }
    }
}

// grid: one workgroup per CU, SB_THREADS threads.  gu: this call's sums;
// gz (zn floats): the other buffer, cleared for the next call.
__global__ __launch_bounds__(SB_THREADS, 1) void k_small_down(Layer L, Work W, const float *__restrict__ gu,
                                                              float *__restrict__ gz, int zn, int n,
                                                              float *__restrict__ out) {
    __shared__ uint2 QT[256 * QT_REPL];
    __shared__ __align__(16) uint8_t hr[2 * SMALL_MAX_TOK * SB_HP];
    __shared__ __align__(16) uint8_t hsh[SMALL_MAX_TOK * SB_SP];
    __shared__ SbRoute R;
    __shared__ int offs[MAX_EXPERT + 1];
    __shared__ uint32_t hmax[3 * SMALL_MAX_TOK];  // per-row maxima: routed slots u0, u0 + 1, shared
    __shared__ float hsc[2 * SMALL_MAX_TOK], shsc[SMALL_MAX_TOK];
    const int tid = threadIdx.x, wave = tid >> 6;
    const int E = L.n_embd, F = L.n_ff, k = L.top_k;
    // the other sum buffer, cleared for the next call (its last reader was the
    // previous call's down kernel, which has completed)
    {
        const int z0 = (int)((int64_t)(zn >> 2) * blockIdx.x / gridDim.x);
        const int z1 = (int)((int64_t)(zn >> 2) * (blockIdx.x + 1) / gridDim.x);
        for (int z = z0 + tid; z < z1; z += SB_THREADS) reinterpret_cast<float4 *>(gz)[z] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (tid < 3 * SMALL_MAX_TOK) hmax[tid] = 0u;
    sb_read_route(L, W, n, R, offs, false);
    const int TE = E >> 4, U = R.U;
    const int nr = U * TE, ns = L.n_shared ? TE * (F >> 8) : 0;
    int g0, g1;
    sb_range(nr, SB_DN_COST_ROUTED, ns, SB_DN_COST_SHARED, g0, g1);
    int i = g0 + wave;
    // the routed slots (at most two: a range is shorter than a slot's units,
    // which the grid size guarantees) and the shared K parts (at most two) of
    // this workgroup's units, whose h vectors are staged
    const int u0 = g0 < nr ? g0 / TE : 0, u1 = g0 < nr ? (min(g1, nr) - 1) / TE : -1;
    const int kp0 = g1 > nr ? (max(g0, nr) - nr) / TE : 0, kp1 = g1 > nr ? (g1 - 1 - nr) / TE : -1;
    const bool rt = g0 < g1 && u1 >= u0, sh = g0 < g1 && kp1 >= kp0;
    const int shk0 = 256 * kp0, shnk = 256 * (kp1 - kp0 + 1);
    // the h vectors are staged before the first unit's weights are requested:
    // behind every CU's weight requests the sums would take several times as
    // long to arrive
    SbStage st;
    q2k_build_table(QT, tid, SB_THREADS);
    if (rt) {
        sb_stage_issue(gu, F, R, u0, k, R.cnt[u0], 0, F, st);
        sb_stage_finish(R.cnt[u0], F, st, hr, SB_HP, hsc, hmax);
    } else if (sh) {
        sb_stage_issue(gu, F, R, -1, k, n, shk0, shnk, st);
        sb_stage_finish(n, shnk, st, hsh, SB_SP, shsc, hmax + 2 * SMALL_MAX_TOK);
    }
    if (rt && u1 > u0) {
        sb_stage_issue(gu, F, R, u1, k, R.cnt[u1], 0, F, st);
        sb_stage_finish(R.cnt[u1], F, st, hr + SMALL_MAX_TOK * SB_HP, SB_HP, hsc + SMALL_MAX_TOK,
                        hmax + SMALL_MAX_TOK);
    }
    if (rt && sh) {
        sb_stage_issue(gu, F, R, -1, k, n, shk0, shnk, st);
        sb_stage_finish(n, shnk, st, hsh, SB_SP, shsc, hmax + 2 * SMALL_MAX_TOK);
    }
    SbDW wa, wb;
    sb_dn_load(L, R, i, 0, nr, TE, i >= g1, wa);
    __syncthreads();
    // the wave's units by halves, as in k_small_gateup
    for (; i < g1; i += SB_WAVES) {
        sb_dn_load(L, R, i, 1, nr, TE, false, wb);
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        sb_dn_compute(L, R, QT, hr, u0, hsh, kp0, i, 0, nr, TE, n, wa, acc);
        const int nx = i + SB_WAVES;
        sb_dn_load(L, R, nx, 0, nr, TE, nx >= g1, wa);
        sb_dn_compute(L, R, QT, hr, u0, hsh, kp0, i, 1, nr, TE, n, wb, acc);
        sb_dn_store(L, R, hsc, u0, shsc, i, nr, TE, n, acc, out);
    }
}

// ---------------------------------------------------------------- launchers
int small_grid() {
    int dev = 0, ncu = 0, g = 0, d = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&g, reinterpret_cast<const void *>(&k_small_gateup),
                                                     SB_THREADS, 0) != hipSuccess || g < 1)
        return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&d, reinterpret_cast<const void *>(&k_small_down), SB_THREADS,
                                                     0) != hipSuccess || d < 1)
        return 0;
    return ncu;
}

size_t small_sum_floats(const Layer &L) { return (size_t)SMALL_MAX_TOK * (L.top_k + 1) * 2 * L.n_ff; }

hipError_t launch_small_gateup(const Layer &L, const Work &W, const void *x, int n_tok, float *gu, int grid,
                               hipStream_t s) {
    hipLaunchKernelGGL(k_small_gateup, dim3(grid), dim3(SB_THREADS), 0, s, L, W, static_cast<const uint16_t *>(x),
                       n_tok, gu);
    return hipGetLastError();
}

hipError_t launch_small_down(const Layer &L, const Work &W, const float *gu, float *gz, int n_tok, float *out,
                             int grid, hipStream_t s) {
    hipLaunchKernelGGL(k_small_down, dim3(grid), dim3(SB_THREADS), 0, s, L, W, gu, gz, (int)small_sum_floats(L),
                       n_tok, out);
    return hipGetLastError();
}

}  // namespace ds4
