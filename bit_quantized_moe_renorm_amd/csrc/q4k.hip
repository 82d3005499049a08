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
// Decode (few tokens): dequant-fused GEMVs.  A lane covers 64 weights of a row
// (a quarter block: two sub-blocks, 32 qs bytes), one sub-block at a time; per
// sub-block it forms sum q x in fp32 (the quants convert exactly) and applies
// d sc * sum q x - dmin m * sum x, the min term through the per-sub-block sums
// of the input vector.  Weights are loaded once per expert and reused for all
// of that expert's tokens, which are taken one at a time.
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

// One sub-block (32 weights) of a lane's quarter block: sum q x over its 16
// quant bytes qw (weight 2 b + 8 wd in the low nibble of byte b of word wd,
// its neighbour in the high nibble) and 32 input values v.
__device__ __forceinline__ float q4k_sub_dot(const uint4 &qw, const float *v) {
    const uint32_t Q[4] = {qw.x, qw.y, qw.z, qw.w};
    float dot = 0.0f;
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
        const uint32_t lo = Q[wd] & 0x0F0F0F0Fu, hi = (Q[wd] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            dot = fmaf((float)((lo >> (8 * b)) & 0xFFu), v[8 * wd + 2 * b], dot);
            dot = fmaf((float)((hi >> (8 * b)) & 0xFFu), v[8 * wd + 2 * b + 1], dot);
        }
    }
    return dot;
}

// A lane's quarter block (sub-blocks 2 qq and 2 qq + 1) is taken one
// sub-block at a time, so a lane holds 32 input values, not 64: per row, r
// accumulates sc * dot and mn accumulates m * (sum of the 32 inputs), and the
// row's value is d r - dmin mn.
struct Q4Acc {
    float r, mn;
};
__device__ __forceinline__ void q4k_sub_acc(Q4Acc &a, const uint4 &meta, const uint4 &qw, int s, const float *v,
                                            float vs) {
    const float dot = q4k_sub_dot(qw, v);
    a.r = fmaf((float)q4k_field(meta, s), dot, a.r);
    a.mn = fmaf((float)q4k_field(meta, 8 + s), vs, a.mn);
}
__device__ __forceinline__ float q4k_acc_value(const Q4Acc &a, const uint4 &meta) {
    const float d = half_to_f32((uint16_t)(meta.x & 0xFFFFu)), dmin = half_to_f32((uint16_t)(meta.x >> 16));
    return d * a.r - dmin * a.mn;
}

// 32 input values of a lane (fp32 or bf16 source) and their sum, in order.
template <bool XBF16>
__device__ __forceinline__ void q4_load_half(const void *src, int64_t off, float *v, float &vs) {
    if (XBF16) {
        const uint4 *p = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(src) + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 r = p[i];
            const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
                v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
            }
        }
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(src) + off);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 r = p[i];
            v[4 * i] = r.x, v[4 * i + 1] = r.y, v[4 * i + 2] = r.z, v[4 * i + 3] = r.w;
        }
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) a += v[i];
    vs = a;
}

constexpr int Q4_WAVES = 4;
constexpr int Q4_GU_NR = 2;  // gate/up rows per lane slot (each row: gate and up)
constexpr int Q4_DN_NR = 4;  // down rows per lane slot

// Routed gate/up: blockIdx.y = active expert slot, blockIdx.x = tile of rows.
// h = SiLU(gate) up of every token of the expert -> hbuf (fp32, slot rows).
template <bool XBF16>
__global__ __launch_bounds__(64 * Q4_WAVES) void k_q4_gateup_routed(Layer L, Work W, const void *__restrict__ x) {
    const int u = blockIdx.y;
    if (u >= W.active[0]) return;
    const int e = W.active[1 + u];
    const int es = expert_slot(L, e);  // the slot holding its weights
    const int beg = W.offsets[e], m = W.offsets[e + 1] - beg;
    const int E = L.n_embd, F = L.n_ff, k = L.top_k, nbe = L.nbe;
    const int lpr = E >> 6, rpw = 64 / lpr;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & (lpr - 1);
    const int rows_per_wave = Q4_GU_NR * rpw;
    const int f0 = (blockIdx.x * Q4_WAVES + wave) * rows_per_wave + lane / lpr;
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
    for (int i = 0; i < m; ++i) {
        const int q = W.list[beg + i];
#pragma unroll
        for (int r = 0; r < Q4_GU_NR; ++r)
            keep_packed(qg[r][0]), keep_packed(qg[r][1]), keep_packed(qu[r][0]), keep_packed(qu[r][1]),
                keep_packed(mg[r]), keep_packed(mu[r]);
        Q4Acc ag[Q4_GU_NR], au[Q4_GU_NR];
#pragma unroll
        for (int r = 0; r < Q4_GU_NR; ++r) ag[r] = au[r] = Q4Acc{0.0f, 0.0f};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            float v[32], vs;
            q4_load_half<XBF16>(x, (int64_t)(q / k) * E + 64 * c + 32 * hh, v, vs);
#pragma unroll
            for (int r = 0; r < Q4_GU_NR; ++r) {
                q4k_sub_acc(ag[r], mg[r], qg[r][hh], 2 * (c & 3) + hh, v, vs);
                q4k_sub_acc(au[r], mu[r], qu[r][hh], 2 * (c & 3) + hh, v, vs);
            }
        }
#pragma unroll
        for (int r = 0; r < Q4_GU_NR; ++r) {
            const int f = f0 + r * rpw;
            // the row's sums in the last lane of its group, by DPP
            const float g = group_sum_last(q4k_acc_value(ag[r], mg[r]), lpr);
            const float uu = group_sum_last(q4k_acc_value(au[r], mu[r]), lpr);
            if (c == lpr - 1 && f < F) W.hbuf[(int64_t)q * F + f] = q4_silu(g) * uu;
        }
    }
}

// Routed down + weighted scatter-add into the residual: blockIdx.y = active
// expert slot.
__global__ __launch_bounds__(64 * Q4_WAVES) void k_q4_down_routed(Layer L, Work W, float *__restrict__ out) {
    const int u = blockIdx.y;
    if (u >= W.active[0]) return;
    const int e = W.active[1 + u];
    const int es = expert_slot(L, e);  // the slot holding its weights
    const int beg = W.offsets[e], m = W.offsets[e + 1] - beg;
    const int E = L.n_embd, F = L.n_ff, k = L.top_k, nbf = L.nbf;
    const int lpr = F >> 6, rpw = 64 / lpr;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & (lpr - 1);
    const int rows_per_wave = Q4_DN_NR * rpw;
    const int r0 = (blockIdx.x * Q4_WAVES + wave) * rows_per_wave + lane / lpr;
    uint4 md[Q4_DN_NR], qd[Q4_DN_NR][2];
#pragma unroll
    for (int r = 0; r < Q4_DN_NR; ++r) {
        const int row = min(r0 + r * rpw, E - 1);
        const int64_t blk = ((int64_t)es * E + row) * nbf + (c >> 2);
        const uint8_t *p = L.q4_qs[2] + blk * 128 + 32 * (c & 3);
        qd[r][0] = ld_nt16(p), qd[r][1] = ld_nt16(p + 16);
        md[r] = ld_nt16(L.q4_meta[2] + blk);
    }
    for (int i = 0; i < m; ++i) {
        const int q = W.list[beg + i];
        const float wgt = W.w[q];
#pragma unroll
        for (int r = 0; r < Q4_DN_NR; ++r) keep_packed(qd[r][0]), keep_packed(qd[r][1]), keep_packed(md[r]);
        Q4Acc ad[Q4_DN_NR];
#pragma unroll
        for (int r = 0; r < Q4_DN_NR; ++r) ad[r] = Q4Acc{0.0f, 0.0f};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            float v[32], vs;
            q4_load_half<false>(W.hbuf, (int64_t)q * F + 64 * c + 32 * hh, v, vs);
#pragma unroll
            for (int r = 0; r < Q4_DN_NR; ++r) q4k_sub_acc(ad[r], md[r], qd[r][hh], 2 * (c & 3) + hh, v, vs);
        }
#pragma unroll
        for (int r = 0; r < Q4_DN_NR; ++r) {
            const int row = r0 + r * rpw;
            const float y = group_sum_last(q4k_acc_value(ad[r], md[r]), lpr);
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
