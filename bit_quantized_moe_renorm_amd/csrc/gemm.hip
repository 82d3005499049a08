// gemm.hip - batched path (prefill and batches beyond the GEMV limit): the
// routed and shared expert projections as grouped MFMA GEMMs with the weight
// decode fused into the B-operand load.
//
// Operand roles (v_mfma_f32_16x16x32_{f16,bf16}): A = 16 tokens x 32 K from an
// LDS stage, B = 32 K x 16 weight rows decoded in registers, C = 16 tokens x 16
// rows.  Lane l holds B column l % 16 (one weight row) and K 8(l/16)..+8, which
// is exactly one 8-weight codebook group of an IQ2 sub-block, and C rows
// 4(l/16)..+3 of that same column, so every per-row factor (block scale d,
// sub-block scale, Q2_K d / dmin) is lane-local.
//
// Exactness of the decoded operands ("Redis 作者出手！ds4...", section 2.3):
//   IQ2 gate/up: B = +-(2c+1)(2ls+1), integers <= 217, exact in fp16; the fp16
//     block scale d and the format's constant 1/64 are applied to the fp32
//     partial sum of each 256-K block.
//   Q2_K down:   B = sc * q (<= 45, exact); the block's d multiplies that sum and
//     dmin multiplies the min term sum_s m_s * hsum_s, computed by a 16x16x16
//     MFMA from per-16-row sums of h written by the gate/up epilogue.
// Activations are rounded to fp16 for the routed MFMAs (x and h); overflow of
// the fp16 range turns into inf in the output rather than a silent error.  The
// shared expert keeps its bf16 weights and takes bf16 activations split into a
// high and a low part (two MFMAs), so its only rounding is fp32 accumulation.
#include "common.h"
#include "iq2_tables.h"

#include <algorithm>

namespace ds4 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int CH_TOK = 64;                     // tokens (routed: slots) per chunk
constexpr int STG_PITCH = 80;                  // LDS stage row: 32 16-bit values + 16 B pad
constexpr int STG_BYTES = CH_TOK * STG_PITCH;  // one K-chunk of A for a chunk of tokens
constexpr int GU_ROWS = 128;                   // n_ff rows per gate/up workgroup (32 per wave)
constexpr int DN_ROWS = 256;                   // n_embd rows per down workgroup (64 per wave)
constexpr int PF = 4;                          // prefetch distance in K-chunks

bool gemm_enabled() { return true; }

int gemm_max_chunks(int n_tok, int NE, int k) {
    const int nq = n_tok * k;
    return min(NE, nq) + (nq + CH_TOK - 1) / CH_TOK;
}

__device__ __forceinline__ floatx4 mfma_f16(half8 a, half8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_bf16(uint4 a, uint4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ half8 as_half8(uint4 v) { return __builtin_bit_cast(half8, v); }

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// Sum over the 16 lanes that share l / 16 (the 16 weight rows of one C column block).
__device__ __forceinline__ float row16_sum(float v) {
    v += __shfl_xor(v, 8, 16);
    v += __shfl_xor(v, 4, 16);
    v += __shfl_xor(v, 2, 16);
    v += __shfl_xor(v, 1, 16);
    return v;
}

// ---------------------------------------------------------------- routing -> chunks
// Splits every expert's token list into chunks of at most CH_TOK slots:
// chunk = (expert, first list position, count), experts ascending.
__global__ __launch_bounds__(256) void k_build_chunks(int NE, Work W) {
    __shared__ int wsum[4];
    const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
    int beg = 0, m = 0;
    if (e < NE) {
        beg = W.offsets[e];
        m = W.offsets[e + 1] - beg;
    }
    const int nc = (m + CH_TOK - 1) / CH_TOK;
    int v = nc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int t = __shfl_up(v, off, 64);
        if (lane >= off) v += t;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    int pre = 0;
    for (int w = 0; w < wave; ++w) pre += wsum[w];
    const int start = pre + v - nc;
    for (int i = 0; i < nc; ++i)
        W.chunks[start + i] = make_int4(e, beg + i * CH_TOK, min(CH_TOK, m - i * CH_TOK), 0);
    if (e == 255) *W.nchunks = pre + v;
}

// ---------------------------------------------------------------- activation copies
// x (bf16 or fp32) -> fp16 for the routed GEMMs; for fp32 x also the bf16 high
// and low parts used by the shared expert.
template <bool XBF16>
__global__ __launch_bounds__(256) void k_prep_x(const void *__restrict__ x, int64_t n, uint16_t *__restrict__ x16,
                                                uint16_t *__restrict__ xhi, uint16_t *__restrict__ xlo) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        float v;
        if (XBF16) {
            v = bf16_to_f32(static_cast<const uint16_t *>(x)[i]);
        } else {
            v = static_cast<const float *>(x)[i];
            const uint16_t hi = f32_to_bf16_rne(v);
            xhi[i] = hi;
            xlo[i] = f32_to_bf16_rne(v - bf16_to_f32(hi));
        }
        x16[i] = f16_bits(v);
    }
}

// ---------------------------------------------------------------- LDS stage helpers
// The stage holds one K-chunk (32 values, 64 bytes) of A for CH_TOK token rows;
// thread t moves 16 bytes: row t / 4, quarter t % 4.
__device__ __forceinline__ void stage_put(uint8_t *stg, int tid, uint4 v) {
    *reinterpret_cast<uint4 *>(stg + (tid >> 2) * STG_PITCH + (tid & 3) * 16) = v;
}
// A fragment of token tile i: lane (rl, grp) reads row 16 i + rl, K 8 grp..+8.
__device__ __forceinline__ uint4 stage_get(const uint8_t *stg, int i, int rl, int grp) {
    return *reinterpret_cast<const uint4 *>(stg + (16 * i + rl) * STG_PITCH + grp * 16);
}

// ---------------------------------------------------------------- routed gate/up
// grid: (n_ff / GU_ROWS, max chunks).  Wave w covers n_ff rows f0..f0+31 of
// both gate and up (B fragments: gate f0, gate f0+16, up f0, up f0+16) for all
// tokens of the chunk (up to 4 token tiles), over the whole n_embd.
__global__ __launch_bounds__(256, 2) void k_gemm_gateup_routed(Layer L, Work W) {
    const int c = blockIdx.y;
    if (c >= *W.nchunks) return;
    const int4 ch = W.chunks[c];
    const int e = ch.x, beg = ch.y, cnt = ch.z;
    __shared__ uint4 T[256 * IQ2_REPL];
    __shared__ __align__(16) uint8_t stg[2][STG_BYTES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rl = lane & 15, grp = lane >> 4;
    const int E = L.n_embd, F = L.n_ff, k = L.top_k, nbe = L.nbe;
    const int nt = (cnt + 15) >> 4;
    const int nkc = E / 32;

    // A loader: token row tid / 4 of the chunk
    const int sr = tid >> 2;
    const uint16_t *xrow = nullptr;
    if (sr < cnt) xrow = W.x16 + (int64_t)(W.list[beg + sr] / k) * E + 8 * (tid & 3);

    const int f0 = blockIdx.x * GU_ROWS + wave * 32;
    const uint2 *wq[4];
    const uint16_t *wd[4];
#pragma unroll
    for (int fi = 0; fi < 4; ++fi) {
        const int m = fi >> 1, f = f0 + 16 * (fi & 1) + rl;
        const int64_t rb = ((int64_t)e * F + f) * nbe;
        wq[fi] = reinterpret_cast<const uint2 *>(L.iq2_qs[m] + rb * 64);  // K-chunk kc: wq[fi][kc]
        wd[fi] = L.iq2_d[m] + rb;
    }

    uint4 xv[PF];
    uint2 wr[PF][4];
    const uint4 z4 = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < PF; ++s) {
        xv[s] = (xrow && s < nkc) ? *reinterpret_cast<const uint4 *>(xrow + 32 * s) : z4;
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) wr[s][fi] = (s < nkc) ? wq[fi][s] : make_uint2(0, 0);
    }
    iq2_build_lut<true>(T, L.codebook, tid, 256);
    stage_put(stg[0], tid, xv[0]);
    xv[0] = (xrow && PF < nkc) ? *reinterpret_cast<const uint4 *>(xrow + 32 * PF) : z4;
    __syncthreads();

    floatx4 acc[4][4], blk[4][4];
    const floatx4 zf = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) acc[i][fi] = zf, blk[i][fi] = zf;

    for (int bi = 0; bi < nbe; ++bi) {
        float dsc[4];
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) dsc[fi] = half_to_f32(wd[fi][bi]) * 0.015625f;  // d / 64
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
            const int kc = bi * 8 + cc;
            const int sl = cc & (PF - 1);
            const uint8_t *cur = stg[kc & 1];
            // decode the four B fragments of this K-chunk
            half8 b[4];
#pragma unroll
            for (int fi = 0; fi < 4; ++fi) {
                const uint32_t ib = wr[sl][fi].x, sw = wr[sl][fi].y;
                const uint4 lv = iq2_group_levels(T, (ib >> (8 * grp)) & 0xFFu, (sw >> (7 * grp)) & 0x7Fu, rl);
                const _Float16 s = (_Float16)(float)(2u * (sw >> 28) + 1u);
                b[fi] = as_half8(lv) * s;
            }
            // refill the weight ring for K-chunk kc + PF
#pragma unroll
            for (int fi = 0; fi < 4; ++fi) wr[sl][fi] = (kc + PF < nkc) ? wq[fi][kc + PF] : make_uint2(0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i < nt) {
                    const half8 a = as_half8(stage_get(cur, i, rl, grp));
#pragma unroll
                    for (int fi = 0; fi < 4; ++fi) blk[i][fi] = mfma_f16(a, b[fi], cc == 0 ? zf : blk[i][fi]);
                }
            }
            // stage K-chunk kc + 1 (loaded PF - 1 chunks ago) into the other buffer
            const int sn = (cc + 1) & (PF - 1);
            if (kc + 1 < nkc) {
                stage_put(stg[(kc + 1) & 1], tid, xv[sn]);
                xv[sn] = (xrow && kc + 1 + PF < nkc) ? *reinterpret_cast<const uint4 *>(xrow + 32 * (kc + 1 + PF)) : z4;
            }
            __syncthreads();
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (i < nt)
#pragma unroll
                for (int fi = 0; fi < 4; ++fi) acc[i][fi] += dsc[fi] * blk[i][fi];
    }

    // epilogue: h = silu(gate) * up -> fp16 slot rows; per-16-row sums for the Q2_K min term
    const int FS = F / 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i >= nt) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int tt = 16 * i + 4 * grp + v;
            const int q = (tt < cnt) ? W.list[beg + tt] : -1;
#pragma unroll
            for (int fp = 0; fp < 2; ++fp) {
                const float h = silu(acc[i][fp][v]) * acc[i][fp + 2][v];
                const uint16_t hb = f16_bits(h);
                const float hs = row16_sum(half_to_f32(hb));
                const int f = f0 + 16 * fp;
                if (q >= 0) {
                    W.hbuf16[(int64_t)q * F + f + rl] = hb;
                    if (rl == 0) W.hsum[(int64_t)q * FS + f / 16] = f16_bits(hs);
                }
            }
        }
    }
}

// ---------------------------------------------------------------- routed down + weighted scatter
// Q2_K B decode: a table of the four 2-bit values of each qs byte as fp16
// (8 bytes per entry), 16 replicas interleaved per entry; lane l reads replica l % 16.
constexpr int QT_REPL = 16;
__device__ __forceinline__ void q2k_build_table(uint2 *QT, int tid, int nthreads) {
    for (int i = tid; i < 256 * QT_REPL; i += nthreads) {
        const uint32_t byte = (uint32_t)i / QT_REPL;
        uint32_t h[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t q = (byte >> (2 * j)) & 3u;
            h[j] = (q == 0) ? 0u : (q == 1) ? 0x3C00u : (q == 2) ? 0x4000u : 0x4200u;
        }
        QT[i] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    }
}

// grid: (n_embd / DN_ROWS, max chunks).  Wave w covers n_embd rows
// r0..r0+63 (4 B fragments) for all tokens of the chunk, over the whole n_ff.
__global__ __launch_bounds__(256, 2) void k_gemm_down_routed(Layer L, Work W, float *__restrict__ out) {
    const int c = blockIdx.y;
    if (c >= *W.nchunks) return;
    const int4 ch = W.chunks[c];
    const int e = ch.x, beg = ch.y, cnt = ch.z;
    __shared__ uint2 QT[256 * QT_REPL];
    __shared__ __align__(16) uint8_t stg[2][STG_BYTES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rl = lane & 15, grp = lane >> 4;
    const int E = L.n_embd, F = L.n_ff, nbf = L.nbf;
    const int nt = (cnt + 15) >> 4;
    const int nkc = F / 32, FS = F / 16;

    const int sr = tid >> 2;
    const uint16_t *hrow = nullptr;
    if (sr < cnt) hrow = W.hbuf16 + (int64_t)W.list[beg + sr] * F + 8 * (tid & 3);
    // A rows of the min-term MFMA: token 16 i + rl of each tile
    const uint16_t *hs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tt = 16 * i + rl;
        hs[i] = (tt < cnt) ? W.hsum + (int64_t)W.list[beg + tt] * FS + 4 * grp : nullptr;
    }

    const int r0 = blockIdx.x * DN_ROWS + wave * 64;
    const uint16_t *wq[4];
    const uint4 *wsc[4];
    const uint32_t *wdd[4];
#pragma unroll
    for (int fi = 0; fi < 4; ++fi) {
        const int64_t rb = ((int64_t)e * E + r0 + 16 * fi + rl) * nbf;
        wq[fi] = reinterpret_cast<const uint16_t *>(L.q2k_qs + rb * 64) + grp;  // K-chunk kc: wq[fi][4 kc]
        wsc[fi] = reinterpret_cast<const uint4 *>(L.q2k_sc + rb * 16);
        wdd[fi] = L.q2k_dd + rb;
    }

    uint4 xv[PF];
    uint16_t wr[PF][4];
    const uint4 z4 = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < PF; ++s) {
        xv[s] = (hrow && s < nkc) ? *reinterpret_cast<const uint4 *>(hrow + 32 * s) : z4;
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) wr[s][fi] = (s < nkc) ? wq[fi][4 * s] : (uint16_t)0;
    }
    q2k_build_table(QT, tid, 256);
    stage_put(stg[0], tid, xv[0]);
    xv[0] = (hrow && PF < nkc) ? *reinterpret_cast<const uint4 *>(hrow + 32 * PF) : z4;
    __syncthreads();

    floatx4 acc[4][4], blk[4][4];
    const floatx4 zf = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) acc[i][fi] = zf, blk[i][fi] = zf;

    for (int bi = 0; bi < nbf; ++bi) {
        uint4 scv[4];
        uint32_t ddv[4];
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) scv[fi] = wsc[fi][bi], ddv[fi] = wdd[fi][bi];
        uint2 hsv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hsv[i] = hs[i] ? *reinterpret_cast<const uint2 *>(hs[i] + 16 * bi) : make_uint2(0, 0);
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
            const int kc = bi * 8 + cc;
            const int sl = cc & (PF - 1);
            const uint8_t *cur = stg[kc & 1];
            half8 b[4];
#pragma unroll
            for (int fi = 0; fi < 4; ++fi) {
                const uint32_t qq = wr[sl][fi];
                const uint2 lo = QT[(qq & 0xFFu) * QT_REPL + rl], hi = QT[(qq >> 8) * QT_REPL + rl];
                // scale nibble of the 16-weight sub-block: byte 2 cc + grp / 2 of the block's scales
                const uint32_t scw = (cc < 2) ? scv[fi].x : (cc < 4) ? scv[fi].y : (cc < 6) ? scv[fi].z : scv[fi].w;
                const uint32_t scb = (scw >> (16 * (cc & 1) + 8 * (grp >> 1))) & 0xFu;
                b[fi] = as_half8(make_uint4(lo.x, lo.y, hi.x, hi.y)) * (_Float16)(float)scb;
            }
#pragma unroll
            for (int fi = 0; fi < 4; ++fi) wr[sl][fi] = (kc + PF < nkc) ? wq[fi][4 * (kc + PF)] : (uint16_t)0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i < nt) {
                    const half8 a = as_half8(stage_get(cur, i, rl, grp));
#pragma unroll
                    for (int fi = 0; fi < 4; ++fi) blk[i][fi] = mfma_f16(a, b[fi], cc == 0 ? zf : blk[i][fi]);
                }
            }
            const int sn = (cc + 1) & (PF - 1);
            if (kc + 1 < nkc) {
                stage_put(stg[(kc + 1) & 1], tid, xv[sn]);
                xv[sn] = (hrow && kc + 1 + PF < nkc) ? *reinterpret_cast<const uint4 *>(hrow + 32 * (kc + 1 + PF)) : z4;
            }
            __syncthreads();
        }
        // min term: sum over the block's 16 sub-blocks of m_s * hsum_s (16x16x16 MFMA, K = sub-blocks)
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) {
            const uint32_t mw = (grp == 0) ? scv[fi].x : (grp == 1) ? scv[fi].y : (grp == 2) ? scv[fi].z : scv[fi].w;
            half4 bm;
#pragma unroll
            for (int j = 0; j < 4; ++j) bm[j] = (_Float16)(float)((mw >> (8 * j + 4)) & 0xFu);
            const float d = half_to_f32((uint16_t)(ddv[fi] & 0xFFFFu));
            const float dmin = half_to_f32((uint16_t)(ddv[fi] >> 16));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i < nt) {
                    const half4 am = __builtin_bit_cast(half4, hsv[i]);
                    const floatx4 mn = __builtin_amdgcn_mfma_f32_16x16x16f16(am, bm, zf, 0, 0, 0);
                    acc[i][fi] += d * blk[i][fi] - dmin * mn;
                }
            }
        }
    }

    // epilogue: out[token][row] += w * y
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i >= nt) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int tt = 16 * i + 4 * grp + v;
            if (tt >= cnt) continue;
            const int q = W.list[beg + tt];
            const float wgt = W.w[q];
            float *orow = out + (int64_t)(q / L.top_k) * E + r0 + rl;
#pragma unroll
            for (int fi = 0; fi < 4; ++fi) atomicAdd(orow + 16 * fi, wgt * acc[i][fi][v]);
        }
    }
}

// ---------------------------------------------------------------- shared expert gate/up
// grid: (n_ff / GU_ROWS, ceil(n_tok / CH_TOK)).  bf16 weights straight from
// memory; A = x as bf16 (SPLIT: high and low bf16 parts of fp32 x).
template <bool SPLIT>
__global__ __launch_bounds__(256, 2) void k_gemm_gateup_shared(Layer L, Work W, const uint16_t *__restrict__ xhi,
                                                               const uint16_t *__restrict__ xlo, int n_tok) {
    const int t0 = blockIdx.y * CH_TOK;
    const int cnt = min(CH_TOK, n_tok - t0);
    __shared__ __align__(16) uint8_t stg[2][2][STG_BYTES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rl = lane & 15, grp = lane >> 4;
    const int E = L.n_embd, F = L.n_ff;
    const int nt = (cnt + 15) >> 4;
    const int nkc = E / 32;
    const int sr = tid >> 2;
    const int64_t xo = (int64_t)(t0 + sr) * E + 8 * (tid & 3);
    const bool xok = sr < cnt;

    const int f0 = blockIdx.x * GU_ROWS + wave * 32;
    const uint4 *wp[4];
#pragma unroll
    for (int fi = 0; fi < 4; ++fi) {
        const uint16_t *base = (fi >> 1) ? L.sh_up : L.sh_gate;
        wp[fi] = reinterpret_cast<const uint4 *>(base + (int64_t)(f0 + 16 * (fi & 1) + rl) * E + 8 * grp);  // kc: wp[fi][4 kc]
    }
    constexpr int SPF = 2;
    uint4 xh[SPF], xl[SPF], wr[SPF][4];
    const uint4 z4 = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < SPF; ++s) {
        xh[s] = (xok && s < nkc) ? *reinterpret_cast<const uint4 *>(xhi + xo + 32 * s) : z4;
        xl[s] = (SPLIT && xok && s < nkc) ? *reinterpret_cast<const uint4 *>(xlo + xo + 32 * s) : z4;
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) wr[s][fi] = (s < nkc) ? wp[fi][4 * s] : z4;
    }
    stage_put(stg[0][0], tid, xh[0]);
    if (SPLIT) stage_put(stg[0][1], tid, xl[0]);
    xh[0] = (xok && SPF < nkc) ? *reinterpret_cast<const uint4 *>(xhi + xo + 32 * SPF) : z4;
    if (SPLIT) xl[0] = (xok && SPF < nkc) ? *reinterpret_cast<const uint4 *>(xlo + xo + 32 * SPF) : z4;
    __syncthreads();

    floatx4 acc[4][4];
    const floatx4 zf = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) acc[i][fi] = zf;

    for (int k0 = 0; k0 < nkc; k0 += SPF) {
#pragma unroll
        for (int s = 0; s < SPF; ++s) {
            const int kc = k0 + s;
            if (kc >= nkc) break;
            uint4 b[4];
#pragma unroll
            for (int fi = 0; fi < 4; ++fi) {
                b[fi] = wr[s][fi];
                wr[s][fi] = (kc + SPF < nkc) ? wp[fi][4 * (kc + SPF)] : z4;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i < nt) {
                    const uint4 a = stage_get(stg[kc & 1][0], i, rl, grp);
#pragma unroll
                    for (int fi = 0; fi < 4; ++fi) acc[i][fi] = mfma_bf16(a, b[fi], acc[i][fi]);
                    if (SPLIT) {
                        const uint4 al = stage_get(stg[kc & 1][1], i, rl, grp);
#pragma unroll
                        for (int fi = 0; fi < 4; ++fi) acc[i][fi] = mfma_bf16(al, b[fi], acc[i][fi]);
                    }
                }
            }
            const int sn = (s + 1) & (SPF - 1);
            if (kc + 1 < nkc) {
                stage_put(stg[(kc + 1) & 1][0], tid, xh[sn]);
                if (SPLIT) stage_put(stg[(kc + 1) & 1][1], tid, xl[sn]);
                xh[sn] = (xok && kc + 1 + SPF < nkc) ? *reinterpret_cast<const uint4 *>(xhi + xo + 32 * (kc + 1 + SPF)) : z4;
                if (SPLIT)
                    xl[sn] = (xok && kc + 1 + SPF < nkc) ? *reinterpret_cast<const uint4 *>(xlo + xo + 32 * (kc + 1 + SPF)) : z4;
            }
            __syncthreads();
        }
    }
    // h = silu(gate) * up, stored as bf16 high and low parts
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i >= nt) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int tt = 16 * i + 4 * grp + v;
            if (tt >= cnt) continue;
#pragma unroll
            for (int fp = 0; fp < 2; ++fp) {
                const float h = silu(acc[i][fp][v]) * acc[i][fp + 2][v];
                const uint16_t hi = f32_to_bf16_rne(h);
                const int64_t o = (int64_t)(t0 + tt) * F + f0 + 16 * fp + rl;
                W.hsh_hi[o] = hi;
                W.hsh_lo[o] = f32_to_bf16_rne(h - bf16_to_f32(hi));
            }
        }
    }
}

// ---------------------------------------------------------------- shared expert down
// grid: (n_embd / DN_ROWS, ceil(n_tok / CH_TOK)).  A = h (high and low bf16
// parts), B = bf16 rows of the shared down matrix; out[token][row] += y.
__global__ __launch_bounds__(256, 2) void k_gemm_down_shared(Layer L, Work W, int n_tok, float *__restrict__ out) {
    const int t0 = blockIdx.y * CH_TOK;
    const int cnt = min(CH_TOK, n_tok - t0);
    __shared__ __align__(16) uint8_t stg[2][2][STG_BYTES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rl = lane & 15, grp = lane >> 4;
    const int E = L.n_embd, F = L.n_ff;
    const int nt = (cnt + 15) >> 4;
    const int nkc = F / 32;
    const int sr = tid >> 2;
    const int64_t ho = (int64_t)(t0 + sr) * F + 8 * (tid & 3);
    const bool hok = sr < cnt;

    const int r0 = blockIdx.x * DN_ROWS + wave * 64;
    const uint4 *wp[4];
#pragma unroll
    for (int fi = 0; fi < 4; ++fi)
        wp[fi] = reinterpret_cast<const uint4 *>(L.sh_down + (int64_t)(r0 + 16 * fi + rl) * F + 8 * grp);
    constexpr int SPF = 2;
    uint4 xh[SPF], xl[SPF], wr[SPF][4];
    const uint4 z4 = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < SPF; ++s) {
        xh[s] = (hok && s < nkc) ? *reinterpret_cast<const uint4 *>(W.hsh_hi + ho + 32 * s) : z4;
        xl[s] = (hok && s < nkc) ? *reinterpret_cast<const uint4 *>(W.hsh_lo + ho + 32 * s) : z4;
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) wr[s][fi] = (s < nkc) ? wp[fi][4 * s] : z4;
    }
    stage_put(stg[0][0], tid, xh[0]);
    stage_put(stg[0][1], tid, xl[0]);
    xh[0] = (hok && SPF < nkc) ? *reinterpret_cast<const uint4 *>(W.hsh_hi + ho + 32 * SPF) : z4;
    xl[0] = (hok && SPF < nkc) ? *reinterpret_cast<const uint4 *>(W.hsh_lo + ho + 32 * SPF) : z4;
    __syncthreads();

    floatx4 acc[4][4];
    const floatx4 zf = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) acc[i][fi] = zf;

    for (int k0 = 0; k0 < nkc; k0 += SPF) {
#pragma unroll
        for (int s = 0; s < SPF; ++s) {
            const int kc = k0 + s;
            if (kc >= nkc) break;
            uint4 b[4];
#pragma unroll
            for (int fi = 0; fi < 4; ++fi) {
                b[fi] = wr[s][fi];
                wr[s][fi] = (kc + SPF < nkc) ? wp[fi][4 * (kc + SPF)] : z4;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i < nt) {
                    const uint4 a = stage_get(stg[kc & 1][0], i, rl, grp);
                    const uint4 al = stage_get(stg[kc & 1][1], i, rl, grp);
#pragma unroll
                    for (int fi = 0; fi < 4; ++fi) {
                        acc[i][fi] = mfma_bf16(a, b[fi], acc[i][fi]);
                        acc[i][fi] = mfma_bf16(al, b[fi], acc[i][fi]);
                    }
                }
            }
            const int sn = (s + 1) & (SPF - 1);
            if (kc + 1 < nkc) {
                stage_put(stg[(kc + 1) & 1][0], tid, xh[sn]);
                stage_put(stg[(kc + 1) & 1][1], tid, xl[sn]);
                xh[sn] = (hok && kc + 1 + SPF < nkc) ? *reinterpret_cast<const uint4 *>(W.hsh_hi + ho + 32 * (kc + 1 + SPF)) : z4;
                xl[sn] = (hok && kc + 1 + SPF < nkc) ? *reinterpret_cast<const uint4 *>(W.hsh_lo + ho + 32 * (kc + 1 + SPF)) : z4;
            }
            __syncthreads();
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i >= nt) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int tt = 16 * i + 4 * grp + v;
            if (tt >= cnt) continue;
            float *orow = out + (int64_t)(t0 + tt) * E + r0 + rl;
#pragma unroll
            for (int fi = 0; fi < 4; ++fi) atomicAdd(orow + 16 * fi, acc[i][fi][v]);
        }
    }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_gemm_gateup(const Layer &L, const Work &W, const void *x, int n_tok, hipStream_t s) {
    const int64_t nx = (int64_t)n_tok * L.n_embd;
    const int pg = (int)std::min<int64_t>((nx + 255) / 256, 4096);
    const bool xb = L.act_dtype == 1;
    if (xb)
        hipLaunchKernelGGL(k_prep_x<true>, dim3(pg), dim3(256), 0, s, x, nx, W.x16, nullptr, nullptr);
    else
        hipLaunchKernelGGL(k_prep_x<false>, dim3(pg), dim3(256), 0, s, x, nx, W.x16, W.xhi, W.xlo);
    hipLaunchKernelGGL(k_build_chunks, dim3(1), dim3(256), 0, s, L.n_expert, W);
    const int mc = gemm_max_chunks(n_tok, L.n_expert, L.top_k);
    hipLaunchKernelGGL(k_gemm_gateup_routed, dim3(L.n_ff / GU_ROWS, mc), dim3(256), 0, s, L, W);
    if (L.n_shared) {
        const uint16_t *xh = xb ? static_cast<const uint16_t *>(x) : W.xhi;
        const dim3 g(L.n_ff / GU_ROWS, (n_tok + CH_TOK - 1) / CH_TOK);
        if (xb)
            hipLaunchKernelGGL(k_gemm_gateup_shared<false>, g, dim3(256), 0, s, L, W, xh, nullptr, n_tok);
        else
            hipLaunchKernelGGL(k_gemm_gateup_shared<true>, g, dim3(256), 0, s, L, W, xh, W.xlo, n_tok);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_down(const Layer &L, const Work &W, int n_tok, float *out, hipStream_t s) {
    const int mc = gemm_max_chunks(n_tok, L.n_expert, L.top_k);
    hipLaunchKernelGGL(k_gemm_down_routed, dim3(L.n_embd / DN_ROWS, mc), dim3(256), 0, s, L, W, out);
    if (L.n_shared)
        hipLaunchKernelGGL(k_gemm_down_shared, dim3(L.n_embd / DN_ROWS, (n_tok + CH_TOK - 1) / CH_TOK), dim3(256), 0, s,
                           L, W, n_tok, out);
    return hipGetLastError();
}

}  // namespace ds4
