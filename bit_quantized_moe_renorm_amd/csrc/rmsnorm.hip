// rmsnorm.hip - unit-gain RMSNorm between stacked MoE layers, in fp64 so that
// the bf16 result is the correctly rounded one: x = bf16(h / sqrt(mean(h^2) + eps)).
#include "common.h"

namespace ds4 {

// fp64 -> bf16 bits, round to nearest even on the 8-bit significand (normal range).
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double v) {
    uint64_t u = __double_as_longlong(v);
    const uint64_t lsb = (u >> 45) & 1ull;
    u += (1ull << 44) - 1ull + lsb;
    u &= ~((1ull << 45) - 1ull);
    const float f = (float)__longlong_as_double(u);  // exact: 8 significant bits
    return (uint16_t)(__float_as_uint(f) >> 16);
}

// Rows of VPT * 1024 floats (16-byte aligned): thread i holds float4s i,
// i + 256, ... in registers, all loaded at once, and divides them after the
// reduction.  Any other shape takes the strided kernel below.
template <int VPT>
__global__ __launch_bounds__(256) void k_rmsnorm_vec(const float *__restrict__ h, int n_embd, double eps,
                                                     uint16_t *__restrict__ x) {
    __shared__ double part[4];
    const int t = blockIdx.x;
    const float4 *row = reinterpret_cast<const float4 *>(h + (int64_t)t * n_embd);
    float4 v[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) v[j] = row[threadIdx.x + 256 * j];
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        ss = fma((double)v[j].x, (double)v[j].x, ss);
        ss = fma((double)v[j].y, (double)v[j].y, ss);
        ss = fma((double)v[j].z, (double)v[j].z, ss);
        ss = fma((double)v[j].w, (double)v[j].w, ss);
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const double tot = part[0] + part[1] + part[2] + part[3];
    const double denom = sqrt(tot / n_embd + eps);
    uint2 *out = reinterpret_cast<uint2 *>(x + (int64_t)t * n_embd);
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const uint32_t a = f64_to_bf16_rne((double)v[j].x / denom), b = f64_to_bf16_rne((double)v[j].y / denom);
        const uint32_t c = f64_to_bf16_rne((double)v[j].z / denom), d = f64_to_bf16_rne((double)v[j].w / denom);
        out[threadIdx.x + 256 * j] = make_uint2(a | (b << 16), c | (d << 16));
    }
}

__global__ __launch_bounds__(256) void k_rmsnorm(const float *__restrict__ h, int n_embd, double eps,
                                                 uint16_t *__restrict__ x) {
    __shared__ double part[4];
    const int t = blockIdx.x;
    const float *row = h + (int64_t)t * n_embd;
    double ss = 0.0;
    for (int i = threadIdx.x; i < n_embd; i += 256) {
        const double v = row[i];
        ss = fma(v, v, ss);
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const double tot = part[0] + part[1] + part[2] + part[3];
    const double denom = sqrt(tot / n_embd + eps);
    for (int i = threadIdx.x; i < n_embd; i += 256) x[(int64_t)t * n_embd + i] = f64_to_bf16_rne((double)row[i] / denom);
}

hipError_t launch_rmsnorm(const float *h, int n_tok, int n_embd, double eps, uint16_t *x, hipStream_t s) {
    const bool vec = n_embd % 1024 == 0 && n_embd <= 4096 && reinterpret_cast<uintptr_t>(h) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(x) % 8 == 0;
    switch (vec ? n_embd / 1024 : 0) {
        case 1: hipLaunchKernelGGL(k_rmsnorm_vec<1>, dim3(n_tok), dim3(256), 0, s, h, n_embd, eps, x); break;
        case 2: hipLaunchKernelGGL(k_rmsnorm_vec<2>, dim3(n_tok), dim3(256), 0, s, h, n_embd, eps, x); break;
        case 3: hipLaunchKernelGGL(k_rmsnorm_vec<3>, dim3(n_tok), dim3(256), 0, s, h, n_embd, eps, x); break;
        case 4: hipLaunchKernelGGL(k_rmsnorm_vec<4>, dim3(n_tok), dim3(256), 0, s, h, n_embd, eps, x); break;
        default: hipLaunchKernelGGL(k_rmsnorm, dim3(n_tok), dim3(256), 0, s, h, n_embd, eps, x); break;
    }
    return hipGetLastError();
}

}  // namespace ds4
