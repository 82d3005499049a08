// repack.hip - create-time repacking of the routed experts into the library
// layout, and the debug decoder that expands a repacked matrix to fp32.
#include "common.h"
#include "iq2_tables.h"

namespace ds4 {

// One thread per 32-weight sub-block: canonical 66-byte blocks -> qs plane (the
// sub-block's 8 canonical bytes, 8-byte aligned) + d plane.
__global__ void k_repack_iq2(const uint8_t *__restrict__ canon, int64_t n_sub, uint8_t *__restrict__ qs,
                             uint16_t *__restrict__ dplane) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_sub) return;
    int64_t b = i >> 3;
    int s = (int)(i & 7);
    const uint8_t *blk = canon + b * 66;
    const uint16_t *sub = reinterpret_cast<const uint16_t *>(blk + 2 + 8 * s);  // 2-byte aligned
    uint32_t D0 = (uint32_t)sub[0] | ((uint32_t)sub[1] << 16);
    uint32_t D1 = (uint32_t)sub[2] | ((uint32_t)sub[3] << 16);
    *reinterpret_cast<uint2 *>(qs + b * 64 + s * 8) = make_uint2(D0, D1);
    if (s == 0) dplane[b] = *reinterpret_cast<const uint16_t *>(blk);
}

// One thread per 84-byte block (4-byte aligned): split into qs / scales / d|dmin planes.
__global__ void k_repack_q2k(const uint8_t *__restrict__ canon, int64_t n_blocks, uint8_t *__restrict__ qs,
                             uint8_t *__restrict__ sc, uint32_t *__restrict__ dd) {
    int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= n_blocks) return;
    const uint32_t *src = reinterpret_cast<const uint32_t *>(canon + b * 84);
    uint32_t *dsc = reinterpret_cast<uint32_t *>(sc + b * 16);
    uint32_t *dqs = reinterpret_cast<uint32_t *>(qs + b * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) dsc[i] = src[i];
#pragma unroll
    for (int i = 0; i < 16; ++i) dqs[i] = src[4 + i];
    dd[b] = src[20];
}

hipError_t launch_repack_iq2(const uint8_t *canon, int64_t n_blocks, uint8_t *qs, uint16_t *d,
                             hipStream_t s) {
    int64_t n_sub = n_blocks * 8;
    int64_t grid = (n_sub + 255) / 256;
    hipLaunchKernelGGL(k_repack_iq2, dim3((unsigned)grid), dim3(256), 0, s, canon, n_sub, qs, d);
    return hipGetLastError();
}

hipError_t launch_repack_q2k(const uint8_t *canon, int64_t n_blocks, uint8_t *qs, uint8_t *sc,
                             uint32_t *dd, hipStream_t s) {
    int64_t grid = (n_blocks + 255) / 256;
    hipLaunchKernelGGL(k_repack_q2k, dim3((unsigned)grid), dim3(256), 0, s, canon, n_blocks, qs, sc, dd);
    return hipGetLastError();
}

// Debug decode of one IQ2 matrix [F][E] to fp32 through the same LDS table and
// sign logic the GEMV kernels use.  One thread per group of 8 weights.
__global__ __launch_bounds__(256) void k_dequant_iq2(const uint8_t *__restrict__ qs, const uint16_t *__restrict__ dpl,
                                                     const uint16_t *__restrict__ codebook, int64_t n_groups,
                                                     float *__restrict__ dst) {
    __shared__ uint4 T[256 * IQ2_REPL];
    iq2_build_lut<false>(T, codebook, threadIdx.x, blockDim.x);
    __syncthreads();
    int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gi >= n_groups) return;
    int64_t blk = gi >> 5;        // 32 groups per block
    int sub = (int)((gi >> 2) & 7);
    int g = (int)(gi & 3);
    const uint32_t *sw = reinterpret_cast<const uint32_t *>(qs + blk * 64 + sub * 8);
    const uint32_t ib = sw[0], signs = sw[1];
    uint4 L = iq2_group_levels(T, (ib >> (8 * g)) & 0xFFu, (signs >> (7 * g)) & 0x7Fu, threadIdx.x & (IQ2_REPL - 1));
    float scale = half_to_f32(dpl[blk]) * (float)(2u * (signs >> 28) + 1u);
    uint32_t lv[4] = {L.x, L.y, L.z, L.w};
    float *o = dst + gi * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = scale * bf16_to_f32((uint16_t)(lv[i] & 0xFFFF)) * 0.015625f;
        o[2 * i + 1] = scale * bf16_to_f32((uint16_t)(lv[i] >> 16)) * 0.015625f;
    }
}

// Debug decode of one Q2_K matrix [E][F]: one thread per weight.
__global__ void k_dequant_q2k(const uint8_t *__restrict__ qs, const uint8_t *__restrict__ sc,
                              const uint32_t *__restrict__ dd, int64_t n, float *__restrict__ dst) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    int64_t blk = i >> 8;
    int w = (int)(i & 255);
    uint32_t q = (qs[blk * 64 + (w >> 2)] >> (2 * (w & 3))) & 3u;
    uint32_t s = sc[blk * 16 + (w >> 4)];
    uint32_t ddv = dd[blk];
    float d = half_to_f32((uint16_t)(ddv & 0xFFFF)), dmin = half_to_f32((uint16_t)(ddv >> 16));
    dst[i] = fmaf(d * (float)(s & 15u), (float)q, -(dmin * (float)(s >> 4)));
}

hipError_t launch_dequant_iq2(const Layer &L, int which, int expert, float *dst, hipStream_t s) {
    int64_t blocks = (int64_t)L.n_ff * L.nbe;
    int64_t n_groups = blocks * 32;
    const uint8_t *qs = L.iq2_qs[which] + (int64_t)expert * blocks * 64;
    const uint16_t *d = L.iq2_d[which] + (int64_t)expert * blocks;
    hipLaunchKernelGGL(k_dequant_iq2, dim3((unsigned)((n_groups + 255) / 256)), dim3(256), 0, s, qs, d,
                       L.codebook, n_groups, dst);
    return hipGetLastError();
}

hipError_t launch_dequant_q2k(const Layer &L, int expert, float *dst, hipStream_t s) {
    int64_t blocks = (int64_t)L.n_embd * L.nbf;
    int64_t n = blocks * 256;
    hipLaunchKernelGGL(k_dequant_q2k, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       L.q2k_qs + (int64_t)expert * blocks * 64, L.q2k_sc + (int64_t)expert * blocks * 16,
                       L.q2k_dd + (int64_t)expert * blocks, n, dst);
    return hipGetLastError();
}

}  // namespace ds4
