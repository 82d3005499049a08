// shared_blas.hip - the shared expert of large calls on hipBLASLt.
//
// The shared expert is a plain bf16 SwiGLU feed-forward applied to every token
// with weight 1 ("ds4 深度实战...", section 3.2: its output is added to the
// routed experts'; section 2.1: it stays at full precision).  For calls of
// many tokens with bf16 activations it is two dense GEMMs, which the library
// GEMM runs at about twice the rate of the grouped kernels' shared-expert
// tiles (measured at 2048 tokens: 69 against 146 us for gate and up).  So:
//   1. gate and up as one GEMM over the adjacent weight planes ([2 n_ff]
//      rows), fp32 output;
//   2. h = SiLU(g) u, split into bf16 high and low parts (h = hi + lo to
//      about 2^-16 relative), as the grouped kernels' epilogue does;
//   3. the down projection as two GEMMs, high part then low part, each added
//      into the fp32 residual (beta = 1).
// Every product of bf16 operands is exact and is accumulated in fp32.
// Calls run in chunks of at most SBLAS_CHUNK tokens (the fp32 gate/up buffer
// is sized for one chunk).
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <new>
#include <utility>

#include "common.h"

namespace ds4 {

struct SharedBlas {
    hipblasLtHandle_t lt = nullptr;
    hipblasLtMatmulDesc_t desc = nullptr;  // op(A) = A^T, op(B) = B, fp32 compute and scale
    hipblasLtMatmulPreference_t pref = nullptr;
    void *ws = nullptr;
    size_t ws_bytes = 0;
    float *gu = nullptr;  // [SBLAS_CHUNK][2 n_ff] fp32
    // the chosen algorithm per (GEMM, token count): 0 gate/up, 1 down
    std::map<std::pair<int, int>, hipblasLtMatmulAlgo_t> algos;
};

namespace {

constexpr size_t SBLAS_WS_BYTES = 32u << 20;

bool ok(hipblasStatus_t s) { return s == HIPBLAS_STATUS_SUCCESS; }

__device__ __forceinline__ float sblas_silu(float g) { return g / (1.0f + __expf(-g)); }

// h = SiLU(gate) * up from the fp32 GEMM output (row t: n_ff gate values, then
// n_ff up values), stored as bf16 high and low parts.
__global__ __launch_bounds__(256) void k_swiglu_split(const float *__restrict__ gu, int64_t n, int F,
                                                      uint16_t *__restrict__ hi, uint16_t *__restrict__ lo) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n * F; i += (int64_t)gridDim.x * 256) {
        const int64_t t = i / F;
        const int f = (int)(i - t * F);
        const float h = sblas_silu(gu[t * 2 * F + f]) * gu[t * 2 * F + F + f];
        const uint16_t h16 = f32_to_bf16_rne(h);
        hi[i] = h16;
        lo[i] = f32_to_bf16_rne(h - bf16_to_f32(h16));
    }
}

// D[m x n] (column-major) = A^T B (+ beta D): A stored column-major k x m
// (lda k), B column-major k x n (ldb k), D column-major m x n (ldd m).
hipblasStatus_t gemm_tn(SharedBlas *S, int which, int m, int n, int k, const void *A, const void *B, float beta,
                        float *D, hipStream_t s) {
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
    hipblasStatus_t st = hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, (uint64_t)k, (uint64_t)m, k);
    if (ok(st)) st = hipblasLtMatrixLayoutCreate(&lb, HIP_R_16BF, (uint64_t)k, (uint64_t)n, k);
    if (ok(st)) st = hipblasLtMatrixLayoutCreate(&ld, HIP_R_32F, (uint64_t)m, (uint64_t)n, m);
    if (ok(st)) {
        auto key = std::make_pair(which, n);
        auto it = S->algos.find(key);
        if (it == S->algos.end()) {
            hipblasLtMatmulHeuristicResult_t res[1];
            int got = 0;
            st = hipblasLtMatmulAlgoGetHeuristic(S->lt, S->desc, la, lb, ld, ld, S->pref, 1, res, &got);
            if (ok(st) && got < 1) st = HIPBLAS_STATUS_NOT_SUPPORTED;
            if (ok(st)) it = S->algos.emplace(key, res[0].algo).first;
        }
        if (ok(st)) {
            const float alpha = 1.0f;
            st = hipblasLtMatmul(S->lt, S->desc, &alpha, A, la, B, lb, &beta, D, ld, D, ld, &it->second, S->ws,
                                 S->ws_bytes, s);
        }
    }
    if (la) hipblasLtMatrixLayoutDestroy(la);
    if (lb) hipblasLtMatrixLayoutDestroy(lb);
    if (ld) hipblasLtMatrixLayoutDestroy(ld);
    return st;
}

}  // namespace

int sblas_create(SharedBlas **out, int n_ff) {
    *out = nullptr;
    SharedBlas *S = new (std::nothrow) SharedBlas();
    if (!S) return -2;
    bool good = ok(hipblasLtCreate(&S->lt));
    good = good && ok(hipblasLtMatmulDescCreate(&S->desc, HIPBLAS_COMPUTE_32F, HIP_R_32F));
    const int32_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    good = good && ok(hipblasLtMatmulDescSetAttribute(S->desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof ta));
    good = good && ok(hipblasLtMatmulDescSetAttribute(S->desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof tb));
    good = good && ok(hipblasLtMatmulPreferenceCreate(&S->pref));
    const uint64_t wsb = SBLAS_WS_BYTES;
    good = good && ok(hipblasLtMatmulPreferenceSetAttribute(S->pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb,
                                                            sizeof wsb));
    if (good && hipMalloc(&S->ws, SBLAS_WS_BYTES) != hipSuccess) S->ws = nullptr, good = false;
    if (good) S->ws_bytes = SBLAS_WS_BYTES;
    if (good && hipMalloc((void **)&S->gu, (size_t)SBLAS_CHUNK * 2 * n_ff * 4) != hipSuccess) S->gu = nullptr, good = false;
    if (!good) {
        hipGetLastError();
        sblas_destroy(S);
        return -1;
    }
    *out = S;
    return 0;
}

void sblas_destroy(SharedBlas *S) {
    if (!S) return;
    if (S->gu) (void)hipFree(S->gu);
    if (S->ws) (void)hipFree(S->ws);
    if (S->pref) hipblasLtMatmulPreferenceDestroy(S->pref);
    if (S->desc) hipblasLtMatmulDescDestroy(S->desc);
    if (S->lt) hipblasLtDestroy(S->lt);
    delete S;
}

hipError_t sblas_gateup(SharedBlas *S, const Layer &L, const Work &W, const void *x, int n_tok, hipStream_t s) {
    const int E = L.n_embd, F = L.n_ff;
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    for (int c0 = 0; c0 < n_tok; c0 += SBLAS_CHUNK) {
        const int n = n_tok - c0 < SBLAS_CHUNK ? n_tok - c0 : SBLAS_CHUNK;
        // gate and up (adjacent planes: [2 F][E] row-major = E x 2F column-major)
        if (!ok(gemm_tn(S, 0, 2 * F, n, E, L.sh_gate, xb + (int64_t)c0 * E, 0.0f, S->gu, s))) return hipErrorUnknown;
        const int64_t nh = (int64_t)n * F;
        const int grid = (int)((nh + 255) / 256 < 4096 ? (nh + 255) / 256 : 4096);
        hipLaunchKernelGGL(k_swiglu_split, dim3(grid), dim3(256), 0, s, S->gu, (int64_t)n, F,
                           W.hsh_hi + (int64_t)c0 * F, W.hsh_lo + (int64_t)c0 * F);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t sblas_down(SharedBlas *S, const Layer &L, const Work &W, int n_tok, float *out, hipStream_t s) {
    const int E = L.n_embd, F = L.n_ff;
    for (int c0 = 0; c0 < n_tok; c0 += SBLAS_CHUNK) {
        const int n = n_tok - c0 < SBLAS_CHUNK ? n_tok - c0 : SBLAS_CHUNK;
        // out[t] += Wd h_hi[t] + Wd h_lo[t]  (Wd [E][F] row-major = F x E column-major)
        float *o = out + (int64_t)c0 * E;
        if (!ok(gemm_tn(S, 1, E, n, F, L.sh_down, W.hsh_hi + (int64_t)c0 * F, 1.0f, o, s))) return hipErrorUnknown;
        if (!ok(gemm_tn(S, 1, E, n, F, L.sh_down, W.hsh_lo + (int64_t)c0 * F, 1.0f, o, s))) return hipErrorUnknown;
    }
    return hipSuccess;
}

}  // namespace ds4
