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
    hipLaunchKernelGGL(k_rmsnorm, dim3(n_tok), dim3(256), 0, s, h, n_embd, eps, x);
    return hipGetLastError();
}

}  // namespace ds4
