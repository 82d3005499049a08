// q4k.hip - routed experts in the Q4_K-style format (the q4 model: "ds4 深度实战...",
// section 2.1, the q2-q4 variant keeps its last 6 layers at q4; "Redis 作者出手！
// ds4...", section 3.1, "Q4 (Q4_K)").  The pages give no layout; the stand-in
// block is 144 bytes per 256 weights:
//   bytes 0-1 fp16 d, 2-3 fp16 dmin; bytes 4-15 sixteen 6-bit fields as a
//   little-endian bit stream (field j at bits 6 j..: the scale sc of
//   sub-block j for j < 8, the min m of sub-block j - 8 for j >= 8; a
//   sub-block is 32 weights); bytes 16-143 the 4-bit quants, weight i in
//   nibble i % 2 of byte 16 + i / 2 (low nibble first).
//   w = d sc q - dmin m
// Library layout per matrix [expert][row][block]: a 16-byte meta plane (the
// block's first 16 bytes: d, dmin, the fields) and a 128-byte qs plane: the
// same bytes, each plane aligned for 128-bit loads.
//
// Decode (few tokens): dequant-fused GEMVs on fp16 dot products
// (v_dot2_f32_f16).  A lane covers 64 weights of a row (a quarter block: two
// sub-blocks, 32 qs bytes), one sub-block at a time.  One byte permute puts
// two quant bytes into the low bytes of an fp16 pair, and one AND-OR turns the
// nibble at bits 4-7 of each half into the fp16 number 1 + q/64 (the low
// nibbles are shifted there first, once per word): normal fp16 operands,
// whose products the dot product keeps to fp32 precision (fp16 subnormals,
// which would need no offset, lose bits in it: measured up to 3e-4 relative
// on gfx950).  The sub-block's dot product is then sum x + (sum q x) / 64,
// and the staged sum of x is subtracted (the offset costs about 3 bits of
// the fp32 result).  The input vector (x for gate/up, h for down) is staged
// once per workgroup in LDS as the matching fp16 pairs under a power-of-two
// scale per 64-value chunk: bf16 x converts exactly, fp32 values are split
// into a high and a low fp16 part (22 bits in all).  Per sub-block the row
// forms d sc sum q x - dmin m sum x, the min term through the sub-block's
// plain fp32 sum of the input.  Weights are loaded once per expert and reused for all of
// that expert's tokens, which are taken one at a time; a token's input is
// requested before the weights, so its staging overlaps their round trip.
#include "common.h"

namespace ds4 {

__device__ __forceinline__ float q4_silu(float z) { return z / (1.0f + expf(-z)); }

// Field j (0..15) of a block's meta (its 96-bit field stream in words y, z, w).
__device__ __forceinline__ uint32_t q4k_field(const uint4 &meta, int j) {
    const int o = 6 * j;
    const uint32_t w0 = (o < 32) ? meta.y : (o < 64) ? meta.z : meta.w;
    const uint32_t w1 = (o < 32) ? meta.z : meta.w;
    const int sh = o & 31;
    const uint64_t pair = (uint64_t)w0 | ((uint64_t)w1 << 32);
    return (uint32_t)(pair >> sh) & 63u;
}

typedef _Float16 q4h2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float q4_dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(q4h2, a), __builtin_bit_cast(q4h2, b), c, false);
}
__device__ __forceinline__ uint32_t q4_pack_f16(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

// One input vector (K <= 4096 values, K a multiple of 64) staged for the
// lanes: chunk c = values 64 c .. 64 c + 63 (lane c of a row), half hh = its
// sub-block of 32 values, word wd = 8 of them.  p[part][hh][wd][c] holds the
// fp16 pairs (v0, v2), (v1, v3), (v4, v6), (v5, v7) of values 64 c + 32 hh +
// 8 wd + 0..7, times 2^-e[c] (part 0 the high fp16 part, part 1 the low one,
// fp32 sources only); consecutive lanes read consecutive 16-byte slots.
// vs[hh][c] is the half's plain fp32 sum and vss[hh][c] the same times
// 2^-e[c].  e[c] puts the chunk's largest magnitude in [2^14, 2^15).
struct Q4X {
    uint4 p[2][2][4][64];
    float vs[2][64], vss[2][64];
    int e[64];
};
// Thread t stages values 16 t .. 16 t + 15 (chunk t / 4, quarter t % 4).  In
// two parts: q4_stage_issue loads them (before the weights, so they return
// first), q4_stage_finish converts and stores.
template <bool BF16>
struct Q4Pre {
    uint4 r[BF16 ? 2 : 4];
};
template <bool BF16>
__device__ __forceinline__ void q4_stage_issue(const void *src, int64_t off, int K, Q4Pre<BF16> &pre) {
    // threads past the vector re-read its last 16 values (not stored)
    const int t = min((int)threadIdx.x, K / 16 - 1);
    const uint4 *p = BF16 ? reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(src) + off + 16 * t)
                          : reinterpret_cast<const uint4 *>(static_cast<const float *>(src) + off + 16 * t);
#pragma unroll
    for (int i = 0; i < (BF16 ? 2 : 4); ++i) pre.r[i] = p[i];
}
template <bool BF16>
__device__ __forceinline__ void q4_stage_finish(int K, const Q4Pre<BF16> &pre, Q4X &X) {
    const int t = threadIdx.x;
    const bool act = 16 * t < K;  // K is a multiple of 64: a chunk's 4 threads agree
    float v[16];
#pragma unroll
    for (int i = 0; i < (BF16 ? 2 : 4); ++i) {
        const uint32_t w[4] = {pre.r[i].x, pre.r[i].y, pre.r[i].z, pre.r[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (BF16) {
                v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
                v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
            } else {
                v[4 * i + j] = __uint_as_float(w[j]);
            }
        }
    }
    float mx = 0.0f, hs = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(v[i])), hs += v[i];
    // the chunk's 4 threads are consecutive lanes: quad maxima by DPP
    mx = fmaxf(mx, dpp_f32<0xB1, 0xF, false>(mx));  // quad_perm [1,0,3,2]
    mx = fmaxf(mx, dpp_f32<0x4E, 0xF, false>(mx));  // quad_perm [2,3,0,1]
    hs += dpp_f32<0xB1, 0xF, false>(hs);            // the half's other thread
    const int ex = (int)((__float_as_uint(mx) >> 23) & 0xFFu) - 127;
    const int e = min(max(ex - 14, -120), 120);
    const int c = t >> 2, qq = t & 3, hh = qq >> 1;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const int wd = 2 * (qq & 1) + w;
        float s[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] = ldexpf(v[8 * w + i], -e);  // exact
        const uint32_t h0 = q4_pack_f16(s[0], s[2]), h1 = q4_pack_f16(s[1], s[3]);
        const uint32_t h2 = q4_pack_f16(s[4], s[6]), h3 = q4_pack_f16(s[5], s[7]);
        if (act) X.p[0][hh][wd][c] = make_uint4(h0, h1, h2, h3);
        if (!BF16) {
            // the low part: what the high part's rounding left
            auto lo = [&](uint32_t hp, float a, float b) {
                const q4h2 hv = __builtin_bit_cast(q4h2, hp);
                return q4_pack_f16(a - (float)hv.x, b - (float)hv.y);
            };
            if (act)
                X.p[1][hh][wd][c] = make_uint4(lo(h0, s[0], s[2]), lo(h1, s[1], s[3]), lo(h2, s[4], s[6]),
                                               lo(h3, s[5], s[7]));
        }
    }
    if (act && (qq & 1) == 0) X.vs[hh][c] = hs, X.vss[hh][c] = ldexpf(hs, -e);
    if (act && qq == 0) X.e[c] = e;
}

// sum (1 + q/64) x over one sub-block (32 weights, quant bytes qw: byte b of
// word wd holds weights 8 wd + 2 b, low nibble, and 8 wd + 2 b + 1, high
// nibble) against the staged pairs xp[wd] (and the low parts xl[wd] when LO),
// in the chunk's scaled units.
// NIB (0x00F000F0: bits 4-7 of each half) and ONE (0x3C003C00: fp16 1.0 in
// each half) come in registers (Q4Masks), so each AND-OR is one VOP3
// instruction rather than an AND and an OR with literal constants.
struct Q4Masks {
    uint32_t nib, one;
    __device__ Q4Masks() : nib(0x00F000F0u), one(0x3C003C00u) { asm volatile("" : "+v"(nib), "+v"(one)); }
};
template <bool LO>
__device__ __forceinline__ float q4_sub_dot2(const uint4 &qw, const uint4 (&xp)[4], const uint4 (&xl)[4],
                                             const Q4Masks &mk) {
    const uint32_t Q[4] = {qw.x, qw.y, qw.z, qw.w};
    const uint32_t NIB = mk.nib, ONE = mk.one;
    float d = 0.0f;
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
        const uint32_t Q4 = Q[wd] << 4;  // each byte's low nibble at its bits 4-7
        // bytes 0, 1 (2, 3) into the low bytes of the halves; then 1 + q/64
        const uint32_t h01 = (__builtin_amdgcn_perm(0u, Q[wd], 0x0C010C00u) & NIB) | ONE;
        const uint32_t h23 = (__builtin_amdgcn_perm(0u, Q[wd], 0x0C030C02u) & NIB) | ONE;
        const uint32_t l01 = (__builtin_amdgcn_perm(0u, Q4, 0x0C010C00u) & NIB) | ONE;
        const uint32_t l23 = (__builtin_amdgcn_perm(0u, Q4, 0x0C030C02u) & NIB) | ONE;
        d = q4_dot2(l01, xp[wd].x, d);
        d = q4_dot2(h01, xp[wd].y, d);
        d = q4_dot2(l23, xp[wd].z, d);
        d = q4_dot2(h23, xp[wd].w, d);
        if (LO) {
            d = q4_dot2(l01, xl[wd].x, d);
            d = q4_dot2(h01, xl[wd].y, d);
            d = q4_dot2(l23, xl[wd].z, d);
            d = q4_dot2(h23, xl[wd].w, d);
        }
    }
    return d;
}

// A lane's quarter block (sub-blocks 2 qq and 2 qq + 1) is taken one
// sub-block at a time: per row, r accumulates sc * (dot - scaled sum of the
// sub-block's inputs) = sc * (sum q x) / 64 in scaled units, mn accumulates
// m * (sum of the sub-block's inputs), and the row's value is
// d r 2^(6 + e) - dmin mn.
struct Q4Acc {
    float r, mn;
};
__device__ __forceinline__ void q4k_sub_acc(Q4Acc &a, const uint4 &meta, int s, float dot, float vss, float vs) {
    a.r = fmaf((float)q4k_field(meta, s), dot - vss, a.r);
    a.mn = fmaf((float)q4k_field(meta, 8 + s), vs, a.mn);
}
__device__ __forceinline__ float q4k_acc_value(const Q4Acc &a, const uint4 &meta, int e) {
    const float d = half_to_f32((uint16_t)(meta.x & 0xFFFFu)), dmin = half_to_f32((uint16_t)(meta.x >> 16));
    return d * ldexpf(a.r, 6 + e) - dmin * a.mn;
}
// The lane's staged pairs of half hh.
template <bool LO>
__device__ __forceinline__ void q4_read_x(const Q4X &X, int hh, int c, uint4 (&xp)[4], uint4 (&xl)[4]) {
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
        xp[wd] = X.p[0][hh][wd][c];
        if (LO) xl[wd] = X.p[1][hh][wd][c];
    }
}

constexpr int Q4_WAVES = 4;
constexpr int Q4_GU_NR = 2;  // gate/up rows per lane slot (each row: gate and up)
constexpr int Q4_DN_NR = 2;  // down rows per lane slot (122 VGPRs: 4 waves per SIMD)

// Routed gate/up: blockIdx.y = active expert slot, blockIdx.x = tile of rows.
// h = SiLU(gate) up of every token of the expert -> hbuf (fp32, slot rows).
template <bool XBF16>
__global__ __launch_bounds__(64 * Q4_WAVES) void k_q4_gateup_routed(Layer L, Work W, const void *__restrict__ x) {
    __shared__ Q4X X;
    const int u = blockIdx.y;
    if (u >= W.active[0]) return;
    const int e = W.active[1 + u];
    const int es = expert_slot(L, e);  // the slot holding its weights
    const int beg = W.offsets[e], m = W.offsets[e + 1] - beg;  // m >= 1 for an active expert
    const int E = L.n_embd, F = L.n_ff, k = L.top_k, nbe = L.nbe;
    const int lpr = E >> 6, rpw = 64 / lpr;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & (lpr - 1);
    const int rows_per_wave = Q4_GU_NR * rpw;
    const int f0 = (blockIdx.x * Q4_WAVES + wave) * rows_per_wave + lane / lpr;
    const int q0 = W.list[beg];
    Q4Pre<XBF16> pre;
    q4_stage_issue<XBF16>(x, (int64_t)(q0 / k) * E, E, pre);
    uint4 mg[Q4_GU_NR], mu[Q4_GU_NR], qg[Q4_GU_NR][2], qu[Q4_GU_NR][2];
#pragma unroll
    for (int r = 0; r < Q4_GU_NR; ++r) {
        // rows past n_ff read row n_ff - 1 (dropped below)
        const int f = min(f0 + r * rpw, F - 1);
        const int64_t blk = ((int64_t)es * F + f) * nbe + (c >> 2);
        const uint8_t *pg = L.q4_qs[0] + blk * 128 + 32 * (c & 3), *pu = L.q4_qs[1] + blk * 128 + 32 * (c & 3);
        qg[r][0] = ld_nt16(pg), qg[r][1] = ld_nt16(pg + 16);
        qu[r][0] = ld_nt16(pu), qu[r][1] = ld_nt16(pu + 16);
        mg[r] = ld_nt16(L.q4_meta[0] + blk);
        mu[r] = ld_nt16(L.q4_meta[1] + blk);
    }
    const Q4Masks mk;
    for (int i = 0; i < m; ++i) {
        const int q = i == 0 ? q0 : W.list[beg + i];
        if (i > 0) q4_stage_issue<XBF16>(x, (int64_t)(q / k) * E, E, pre);
        __syncthreads();  // the previous token's reads of X are over
        q4_stage_finish<XBF16>(E, pre, X);
        __syncthreads();
#pragma unroll
        for (int r = 0; r < Q4_GU_NR; ++r)
            keep_packed(qg[r][0]), keep_packed(qg[r][1]), keep_packed(qu[r][0]), keep_packed(qu[r][1]),
                keep_packed(mg[r]), keep_packed(mu[r]);
        Q4Acc ag[Q4_GU_NR], au[Q4_GU_NR];
#pragma unroll
        for (int r = 0; r < Q4_GU_NR; ++r) ag[r] = au[r] = Q4Acc{0.0f, 0.0f};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            uint4 xp[4], xl[4];
            q4_read_x<!XBF16>(X, hh, c, xp, xl);
            const float vs = X.vs[hh][c], vss = X.vss[hh][c];
            const int s = 2 * (c & 3) + hh;
#pragma unroll
            for (int r = 0; r < Q4_GU_NR; ++r) {
                q4k_sub_acc(ag[r], mg[r], s, q4_sub_dot2<!XBF16>(qg[r][hh], xp, xl, mk), vss, vs);
                q4k_sub_acc(au[r], mu[r], s, q4_sub_dot2<!XBF16>(qu[r][hh], xp, xl, mk), vss, vs);
            }
        }
        const int ec = X.e[c];
#pragma unroll
        for (int r = 0; r < Q4_GU_NR; ++r) {
            const int f = f0 + r * rpw;
            // the row's sums in the last lane of its group, by DPP
            const float g = group_sum_last(q4k_acc_value(ag[r], mg[r], ec), lpr);
            const float uu = group_sum_last(q4k_acc_value(au[r], mu[r], ec), lpr);
            if (c == lpr - 1 && f < F) W.hbuf[(int64_t)q * F + f] = q4_silu(g) * uu;
        }
    }
}

// Routed down + weighted scatter-add into the residual: blockIdx.y = active
// expert slot.  h (fp32) is staged in a high and a low fp16 part.
__global__ __launch_bounds__(64 * Q4_WAVES) void k_q4_down_routed(Layer L, Work W, float *__restrict__ out) {
    __shared__ Q4X X;
    const int u = blockIdx.y;
    if (u >= W.active[0]) return;
    const int e = W.active[1 + u];
    const int es = expert_slot(L, e);  // the slot holding its weights
    const int beg = W.offsets[e], m = W.offsets[e + 1] - beg;  // m >= 1 for an active expert
    const int E = L.n_embd, F = L.n_ff, k = L.top_k, nbf = L.nbf;
    const int lpr = F >> 6, rpw = 64 / lpr;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & (lpr - 1);
    const int rows_per_wave = Q4_DN_NR * rpw;
    const int r0 = (blockIdx.x * Q4_WAVES + wave) * rows_per_wave + lane / lpr;
    const int q0 = W.list[beg];
    Q4Pre<false> pre;
    q4_stage_issue<false>(W.hbuf, (int64_t)q0 * F, F, pre);
    uint4 md[Q4_DN_NR], qd[Q4_DN_NR][2];
#pragma unroll
    for (int r = 0; r < Q4_DN_NR; ++r) {
        const int row = min(r0 + r * rpw, E - 1);
        const int64_t blk = ((int64_t)es * E + row) * nbf + (c >> 2);
        const uint8_t *p = L.q4_qs[2] + blk * 128 + 32 * (c & 3);
        qd[r][0] = ld_nt16(p), qd[r][1] = ld_nt16(p + 16);
        md[r] = ld_nt16(L.q4_meta[2] + blk);
    }
    const Q4Masks mk;
    for (int i = 0; i < m; ++i) {
        const int q = i == 0 ? q0 : W.list[beg + i];
        if (i > 0) q4_stage_issue<false>(W.hbuf, (int64_t)q * F, F, pre);
        const float wgt = W.w[q];
        __syncthreads();  // the previous token's reads of X are over
        q4_stage_finish<false>(F, pre, X);
        __syncthreads();
#pragma unroll
        for (int r = 0; r < Q4_DN_NR; ++r) keep_packed(qd[r][0]), keep_packed(qd[r][1]), keep_packed(md[r]);
        Q4Acc ad[Q4_DN_NR];
#pragma unroll
        for (int r = 0; r < Q4_DN_NR; ++r) ad[r] = Q4Acc{0.0f, 0.0f};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            uint4 xp[4], xl[4];
            q4_read_x<true>(X, hh, c, xp, xl);
            const float vs = X.vs[hh][c], vss = X.vss[hh][c];
            const int s = 2 * (c & 3) + hh;
#pragma unroll
            for (int r = 0; r < Q4_DN_NR; ++r)
                q4k_sub_acc(ad[r], md[r], s, q4_sub_dot2<true>(qd[r][hh], xp, xl, mk), vss, vs);
        }
        const int ec = X.e[c];
#pragma unroll
        for (int r = 0; r < Q4_DN_NR; ++r) {
            const int row = r0 + r * rpw;
            const float y = group_sum_last(q4k_acc_value(ad[r], md[r], ec), lpr);
            if (c == lpr - 1 && row < E) atomicAdd(out + (int64_t)(q / k) * E + row, wgt * y);
        }
    }
}

// Debug decode of one Q4_K matrix [rows][cols] to fp32 through the kernels'
// field and nibble extraction: one thread per weight.
__global__ __launch_bounds__(256) void k_dequant_q4k(const uint8_t *__restrict__ qs, const uint4 *__restrict__ meta,
                                                     int64_t n, float *__restrict__ dst) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int64_t b = i >> 8;
    const int w = (int)(i & 255);
    const uint4 mt = meta[b];
    const int s = w >> 5;
    const uint32_t q = (qs[b * 128 + (w >> 1)] >> (4 * (w & 1))) & 15u;
    const float d = half_to_f32((uint16_t)(mt.x & 0xFFFFu)), dmin = half_to_f32((uint16_t)(mt.x >> 16));
    // d sc q and dmin m are exact in fp32 (11 + 6 + 4 and 11 + 6 significant
    // bits), as is their difference for the formats' value ranges
    dst[i] = d * (float)(q4k_field(mt, s) * q) - dmin * (float)q4k_field(mt, 8 + s);
}

// Canonical 144-byte blocks (16-byte aligned) -> meta plane + qs plane.
__global__ void k_repack_q4k(const uint8_t *__restrict__ canon, int64_t n_blocks, uint4 *__restrict__ meta,
                             uint8_t *__restrict__ qs) {
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= n_blocks) return;
    const uint4 *src = reinterpret_cast<const uint4 *>(canon + b * 144);
    meta[b] = src[0];
    uint4 *dq = reinterpret_cast<uint4 *>(qs + b * 128);
#pragma unroll
    for (int i = 0; i < 8; ++i) dq[i] = src[1 + i];
}

hipError_t launch_repack_q4k(const uint8_t *canon, int64_t n_blocks, uint4 *meta, uint8_t *qs, hipStream_t s) {
    hipLaunchKernelGGL(k_repack_q4k, dim3((unsigned)((n_blocks + 255) / 256)), dim3(256), 0, s, canon, n_blocks,
                       meta, qs);
    return hipGetLastError();
}

hipError_t launch_dequant_q4k(const Layer &L, int which, int expert, float *dst, hipStream_t s) {
    const int64_t rows = which < 2 ? L.n_ff : L.n_embd, cols = which < 2 ? L.n_embd : L.n_ff;
    const int64_t nb = rows * (cols / QK), n = rows * cols;
    const uint8_t *qs = L.q4_qs[which] + (int64_t)expert * nb * 128;
    const uint4 *meta = L.q4_meta[which] + (int64_t)expert * nb;
    hipLaunchKernelGGL(k_dequant_q4k, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, qs, meta, n, dst);
    return hipGetLastError();
}

hipError_t launch_q4_gateup_routed(const Layer &L, const Work &W, const void *x, int n_tok, hipStream_t s) {
    const int slots = min(n_tok * L.top_k, L.n_expert);
    const int rpw = 64 / (L.n_embd >> 6);
    const int rows_wg = Q4_WAVES * Q4_GU_NR * rpw;
    const dim3 grid((L.n_ff + rows_wg - 1) / rows_wg, slots);
    if (L.act_dtype == 1)
        hipLaunchKernelGGL(k_q4_gateup_routed<true>, grid, dim3(64 * Q4_WAVES), 0, s, L, W, x);
    else
        hipLaunchKernelGGL(k_q4_gateup_routed<false>, grid, dim3(64 * Q4_WAVES), 0, s, L, W, x);
    return hipGetLastError();
}

hipError_t launch_q4_down_routed(const Layer &L, const Work &W, int n_tok, float *out, hipStream_t s) {
    const int slots = min(n_tok * L.top_k, L.n_expert);
    const int rpw = 64 / (L.n_ff >> 6);
    const int rows_wg = Q4_WAVES * Q4_DN_NR * rpw;
    const dim3 grid((L.n_embd + rows_wg - 1) / rows_wg, slots);
    hipLaunchKernelGGL(k_q4_down_routed, grid, dim3(64 * Q4_WAVES), 0, s, L, W, out);
    return hipGetLastError();
}

}  // namespace ds4
