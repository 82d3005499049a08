// gemv.hip - decode path (few tokens): dequant-fused GEMVs over the 2-bit experts.
//
// Generation is bandwidth-bound ("ds4 深度实战...", section 5.1), so these
// kernels stream each touched weight byte from HBM once with 128-bit loads and
// decode it in registers:
//   * routed gate/up (IQ2-style): one 64-weight chunk (16 bytes) per lane, the
//     signed codebook levels come from the LDS tables (iq2_tables.h), the dot
//     products use v_dot2_f32_bf16 against x held in registers, the sub-block
//     scale (2ls+1) and the fp16 d are applied per sub-block / per lane, and
//     SiLU(gate) * up is formed in registers;
//   * routed down (Q2_K-style): 64 weights per lane, w = d sc q - dmin m with
//     the min term folded through per-sub-block sums of h;
//   * shared expert (bf16): plain streaming dot products.
// Each routed weight row is read once per expert for all of that expert's
// tokens; the weighted down outputs are added into the residual with fp32
// atomics (the merge of routed and shared outputs, "ds4 深度实战...", section 3.2).
#include "common.h"
#include "iq2_tables.h"

namespace ds4 {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }


// x of one token for a 64-weight chunk: bf16 pairs (32 dwords) or fp32 (64 floats).
template <bool XBF16>
struct XChunk;
template <>
struct XChunk<true> {
    uint32_t v[32];
    __device__ __forceinline__ void load(const void *x, int64_t off) {
        const uint4 *p = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(x) + off);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint4 r = p[i];
            v[4 * i] = r.x, v[4 * i + 1] = r.y, v[4 * i + 2] = r.z, v[4 * i + 3] = r.w;
        }
    }
    // sum over 4 dwords (8 weights) starting at dword o of levels L (4 dwords)
    __device__ __forceinline__ float dot8(uint32_t l0, uint32_t l1, uint32_t l2, uint32_t l3, int o, float s) const {
        s = dot2_bf16(l0, v[o], s);
        s = dot2_bf16(l1, v[o + 1], s);
        s = dot2_bf16(l2, v[o + 2], s);
        s = dot2_bf16(l3, v[o + 3], s);
        return s;
    }
};
template <>
struct XChunk<false> {
    float v[64];
    __device__ __forceinline__ void load(const void *x, int64_t off) {
        const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(x) + off);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float4 r = p[i];
            v[4 * i] = r.x, v[4 * i + 1] = r.y, v[4 * i + 2] = r.z, v[4 * i + 3] = r.w;
        }
    }
    __device__ __forceinline__ float dot8(uint32_t l0, uint32_t l1, uint32_t l2, uint32_t l3, int o, float s) const {
        const uint32_t l[4] = {l0, l1, l2, l3};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s = fmaf(__uint_as_float(l[i] << 16), v[2 * (o + i)], s);
            s = fmaf(__uint_as_float(l[i] & 0xFFFF0000u), v[2 * (o + i) + 1], s);
        }
        return s;
    }
};

// Dot of one lane's 64 IQ2 weights (2 canonical sub-blocks) with x, before the
// fp16 d and the 1/64 of the level and scale encodings.
template <bool XBF16>
__device__ __forceinline__ float iq2_chunk_dot(const uint4 *T, uint4 q, const XChunk<XBF16> &xc, int rep) {
    float acc = 0.0f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
        const uint32_t ib = sb ? q.z : q.x;
        const uint32_t sw = sb ? q.w : q.y;
        float s = 0.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint4 Lv = iq2_group_levels(T, (ib >> (8 * g)) & 0xFFu, (sw >> (7 * g)) & 0x7Fu, rep);
            s = xc.dot8(Lv.x, Lv.y, Lv.z, Lv.w, 16 * sb + 4 * g, s);
        }
        acc = fmaf((float)(2u * (sw >> 28) + 1u), s, acc);
    }
    return acc;
}

constexpr int GU_WAVES = 8;
constexpr int GU_NR = 4;

// Routed gate/up: blockIdx.y = active expert slot, blockIdx.x = tile of rows.
template <bool XBF16>
__global__ __launch_bounds__(512) void k_gemv_gateup_routed(Layer L, Work W, const void *__restrict__ x) {
    __shared__ uint4 T[256 * IQ2_REPL];
    const int U = W.active[0];
    const int u = blockIdx.y;
    if (u >= U) return;
    const int e = W.active[1 + u];
    const int es = expert_slot(L, e);  // the slot holding its weights
    const int beg = W.offsets[e];
    const int m = W.offsets[e + 1] - beg;
    const int E = L.n_embd, F = L.n_ff, k = L.top_k;
    const int lpr = E >> 6, rpw = 64 / lpr;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & (lpr - 1);
    const int rows_per_wave = GU_NR * rpw;
    const int f0 = blockIdx.x * (GU_WAVES * rows_per_wave) + wave * rows_per_wave + lane / lpr;

    uint4 qg[GU_NR], qu[GU_NR];
    float dg[GU_NR], du[GU_NR];
#pragma unroll
    for (int r = 0; r < GU_NR; ++r) {
        const int f = f0 + r * rpw;
        if (f < F) {
            const int64_t rb = ((int64_t)es * F + f) * L.nbe;
            qg[r] = ld_nt16(L.iq2_qs[0] + rb * 64 + c * 16);
            qu[r] = ld_nt16(L.iq2_qs[1] + rb * 64 + c * 16);
            dg[r] = half_to_f32(ld_nt2(L.iq2_d[0] + rb + (c >> 2)));
            du[r] = half_to_f32(ld_nt2(L.iq2_d[1] + rb + (c >> 2)));
        } else {
            qg[r] = qu[r] = make_uint4(0, 0, 0, 0);
            dg[r] = du[r] = 0.0f;
        }
    }
    XChunk<XBF16> xc[GEMV_MAX_TOK];
    int slot[GEMV_MAX_TOK];
#pragma unroll
    for (int i = 0; i < GEMV_MAX_TOK; ++i) {
        slot[i] = 0;
        if (i < m) {
            const int q = W.list[beg + i];
            slot[i] = q;
            xc[i].load(x, (int64_t)(q / k) * E + 64 * c);
        }
    }
    iq2_build_lut<false>(T, L.codebook, threadIdx.x, blockDim.x);
    __syncthreads();
    const int rep = lane & (IQ2_REPL - 1);

#pragma unroll
    for (int r = 0; r < GU_NR; ++r) {
        const int f = f0 + r * rpw;
#pragma unroll
        for (int i = 0; i < GEMV_MAX_TOK; ++i) {
            if (i < m) {
                float g = iq2_chunk_dot<XBF16>(T, qg[r], xc[i], rep) * dg[r];
                float uu = iq2_chunk_dot<XBF16>(T, qu[r], xc[i], rep) * du[r];
                // the row's sums in the last lane of its group, by DPP
                g = group_sum_last(g, lpr) * 0.015625f;
                uu = group_sum_last(uu, lpr) * 0.015625f;
                if (c == lpr - 1 && f < F) W.hbuf[(int64_t)slot[i] * F + f] = silu(g) * uu;
            }
        }
    }
}

// Shared-expert gate/up (bf16 weights), every token.  16-byte chunks: lane l
// takes chunks l, l+64, ... of each row (coalesced 1 KB per wave load).
template <bool XBF16, int MAXT>
__global__ __launch_bounds__(256) void k_gemv_gateup_shared(Layer L, Work W, const void *__restrict__ x, int n_tok) {
    // one row of gate and up per wave: 512 workgroups of 4 waves for n_ff
    // 2048 (two rows per wave, 256 workgroups, measured 12.35 -> 11.33 us
    // for one token)
    constexpr int NR = 1;
    constexpr int WAVES = 4;
    const int E = L.n_embd, F = L.n_ff, k = L.top_k;
    const int nch = E >> 3;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int f0 = (blockIdx.x * WAVES + wave) * NR;
    uint4 wg[NR][8], wu[NR][8];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int ch = lane + 64 * it;
            const int f = f0 + r;
            if (ch < nch && f < F) {
                wg[r][it] = ld_nt16(L.sh_gate + (int64_t)f * E + ch * 8);
                wu[r][it] = ld_nt16(L.sh_up + (int64_t)f * E + ch * 8);
            } else {
                wg[r][it] = wu[r][it] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
        if (t >= n_tok) break;
        float xv[8][8];
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int ch = lane + 64 * it;
            if (ch < nch) {
                if (XBF16) {
                    uint4 r = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(x) + (int64_t)t * E + ch * 8);
                    const uint32_t d[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        xv[it][2 * j] = __uint_as_float(d[j] << 16);
                        xv[it][2 * j + 1] = __uint_as_float(d[j] & 0xFFFF0000u);
                    }
                } else {
                    const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(x) + (int64_t)t * E + ch * 8);
                    float4 a = p[0], b = p[1];
                    xv[it][0] = a.x, xv[it][1] = a.y, xv[it][2] = a.z, xv[it][3] = a.w;
                    xv[it][4] = b.x, xv[it][5] = b.y, xv[it][6] = b.z, xv[it][7] = b.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) xv[it][j] = 0.0f;
            }
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            float g = 0.0f, uu = 0.0f;
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const uint32_t a[4] = {wg[r][it].x, wg[r][it].y, wg[r][it].z, wg[r][it].w};
                const uint32_t b[4] = {wu[r][it].x, wu[r][it].y, wu[r][it].z, wu[r][it].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    g = fmaf(__uint_as_float(a[j] << 16), xv[it][2 * j], g);
                    g = fmaf(__uint_as_float(a[j] & 0xFFFF0000u), xv[it][2 * j + 1], g);
                    uu = fmaf(__uint_as_float(b[j] << 16), xv[it][2 * j], uu);
                    uu = fmaf(__uint_as_float(b[j] & 0xFFFF0000u), xv[it][2 * j + 1], uu);
                }
            }
            g = wave_sum(g);
            uu = wave_sum(uu);
            const int f = f0 + r;
            if (lane == 0 && f < F) W.hbuf[((int64_t)n_tok * k + t) * F + f] = silu(g) * uu;
        }
    }
}

// One lane's 64 Q2_K weights (4 sub-blocks of 16) against h (64 floats) with
// the per-sub-block sums of h precomputed.
__device__ __forceinline__ float q2k_chunk_dot(uint4 qs, uint32_t sc, uint32_t dd, const float *hv, const float *hs) {
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
        B = fmaf((float)(scb >> 4), hs[s], B);
    }
    const float d = half_to_f32((uint16_t)(dd & 0xFFFFu)), dmin = half_to_f32((uint16_t)(dd >> 16));
    return d * A - dmin * B;
}

constexpr int DN_WAVES = 4;
constexpr int DN_NR = 4;

// Routed down + weighted scatter-add: blockIdx.y = active expert slot.
__global__ __launch_bounds__(256) void k_gemv_down_routed(Layer L, Work W, float *__restrict__ out) {
    const int U = W.active[0];
    const int u = blockIdx.y;
    if (u >= U) return;
    const int e = W.active[1 + u];
    const int es = expert_slot(L, e);  // the slot holding its weights
    const int beg = W.offsets[e];
    const int m = W.offsets[e + 1] - beg;
    const int E = L.n_embd, F = L.n_ff, k = L.top_k;
    const int lpr = F >> 6, rpw = 64 / lpr;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & (lpr - 1);
    const int rows_per_wave = DN_NR * rpw;
    const int r0 = blockIdx.x * (DN_WAVES * rows_per_wave) + wave * rows_per_wave + lane / lpr;
    uint4 qs[DN_NR];
    uint32_t sc[DN_NR], dd[DN_NR];
#pragma unroll
    for (int r = 0; r < DN_NR; ++r) {
        const int row = r0 + r * rpw;
        if (row < E) {
            const int64_t rb = ((int64_t)es * E + row) * L.nbf;
            qs[r] = ld_nt16(L.q2k_qs + rb * 64 + c * 16);
            sc[r] = ld_nt4(L.q2k_sc + rb * 16 + c * 4);
            dd[r] = ld_nt4(L.q2k_dd + rb + (c >> 2));
        } else {
            qs[r] = make_uint4(0, 0, 0, 0);
            sc[r] = dd[r] = 0u;
        }
    }
    for (int i = 0; i < m; ++i) {
        const int q = W.list[beg + i];
        const int t = q / k;
        const float wgt = W.w[q];
#pragma unroll
        for (int r = 0; r < DN_NR; ++r) keep_packed(qs[r]), keep_packed(sc[r]), keep_packed(dd[r]);
        float hv[64], hs[4];
        const float4 *hp = reinterpret_cast<const float4 *>(W.hbuf + (int64_t)q * F + 64 * c);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float4 v = hp[j];
            hv[4 * j] = v.x, hv[4 * j + 1] = v.y, hv[4 * j + 2] = v.z, hv[4 * j + 3] = v.w;
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            float a = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) a += hv[16 * s + j];
            hs[s] = a;
        }
#pragma unroll
        for (int r = 0; r < DN_NR; ++r) {
            const int row = r0 + r * rpw;
            float y = q2k_chunk_dot(qs[r], sc[r], dd[r], hv, hs);
            y = group_sum_last(y, lpr);
            if (c == lpr - 1 && row < E) atomicAdd(out + (int64_t)t * E + row, wgt * y);
        }
    }
}

// Shared-expert down (bf16 weights), every token, weight 1.
template <int MAXT>
__global__ __launch_bounds__(256) void k_gemv_down_shared(Layer L, Work W, int n_tok, float *__restrict__ out) {
    constexpr int NR = 2, WAVES = 4;
    const int E = L.n_embd, F = L.n_ff, k = L.top_k;
    const int nch = F >> 3;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r0 = (blockIdx.x * WAVES + wave) * NR;
    uint4 wd[NR][8];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int ch = lane + 64 * it;
            const int row = r0 + r;
            wd[r][it] = (ch < nch && row < E)
                            ? ld_nt16(L.sh_down + (int64_t)row * F + ch * 8)
                            : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
        if (t >= n_tok) break;
        const float *hrow = W.hbuf + ((int64_t)n_tok * k + t) * F;
        float hv[8][8];
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int ch = lane + 64 * it;
            if (ch < nch) {
                const float4 *p = reinterpret_cast<const float4 *>(hrow + ch * 8);
                float4 a = p[0], b = p[1];
                hv[it][0] = a.x, hv[it][1] = a.y, hv[it][2] = a.z, hv[it][3] = a.w;
                hv[it][4] = b.x, hv[it][5] = b.y, hv[it][6] = b.z, hv[it][7] = b.w;
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) hv[it][j] = 0.0f;
            }
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            float y = 0.0f;
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const uint32_t a[4] = {wd[r][it].x, wd[r][it].y, wd[r][it].z, wd[r][it].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    y = fmaf(__uint_as_float(a[j] << 16), hv[it][2 * j], y);
                    y = fmaf(__uint_as_float(a[j] & 0xFFFF0000u), hv[it][2 * j + 1], y);
                }
            }
            y = wave_sum(y);
            const int row = r0 + r;
            if (lane == 0 && row < E) atomicAdd(out + (int64_t)t * E + row, y);
        }
    }
}

hipError_t launch_gemv_gateup_routed(const Layer &L, const Work &W, const void *x, int n_tok, hipStream_t s) {
    const int slots = min(n_tok * L.top_k, L.n_expert);
    const int rpw = 64 / (L.n_embd >> 6);
    const int rows_wg = GU_WAVES * GU_NR * rpw;
    dim3 grid((L.n_ff + rows_wg - 1) / rows_wg, slots);
    if (L.act_dtype == 1)
        hipLaunchKernelGGL(k_gemv_gateup_routed<true>, grid, dim3(64 * GU_WAVES), 0, s, L, W, x);
    else
        hipLaunchKernelGGL(k_gemv_gateup_routed<false>, grid, dim3(64 * GU_WAVES), 0, s, L, W, x);
    return hipGetLastError();
}

hipError_t launch_gemv_gateup_shared(const Layer &L, const Work &W, const void *x, int n_tok, hipStream_t s) {
    const bool bf = L.act_dtype == 1;
    dim3 g2((L.n_ff + 3) / 4);  // 4 waves of one row each
    if (n_tok == 1) {
        if (bf) hipLaunchKernelGGL((k_gemv_gateup_shared<true, 1>), g2, dim3(256), 0, s, L, W, x, n_tok);
        else hipLaunchKernelGGL((k_gemv_gateup_shared<false, 1>), g2, dim3(256), 0, s, L, W, x, n_tok);
    } else {
        if (bf) hipLaunchKernelGGL((k_gemv_gateup_shared<true, GEMV_MAX_TOK>), g2, dim3(256), 0, s, L, W, x, n_tok);
        else hipLaunchKernelGGL((k_gemv_gateup_shared<false, GEMV_MAX_TOK>), g2, dim3(256), 0, s, L, W, x, n_tok);
    }
    return hipGetLastError();
}

hipError_t launch_gemv_down_routed(const Layer &L, const Work &W, int n_tok, float *out, hipStream_t s) {
    const int slots = min(n_tok * L.top_k, L.n_expert);
    const int rpw = 64 / (L.n_ff >> 6);
    const int rows_wg = DN_WAVES * DN_NR * rpw;
    dim3 grid((L.n_embd + rows_wg - 1) / rows_wg, slots);
    hipLaunchKernelGGL(k_gemv_down_routed, grid, dim3(64 * DN_WAVES), 0, s, L, W, out);
    return hipGetLastError();
}

hipError_t launch_gemv_down_shared(const Layer &L, const Work &W, int n_tok, float *out, hipStream_t s) {
    dim3 g2((L.n_embd + 7) / 8);
    if (n_tok == 1) hipLaunchKernelGGL(k_gemv_down_shared<1>, g2, dim3(256), 0, s, L, W, n_tok, out);
    else hipLaunchKernelGGL(k_gemv_down_shared<GEMV_MAX_TOK>, g2, dim3(256), 0, s, L, W, n_tok, out);
    return hipGetLastError();
}

}  // namespace ds4
