// common.h - internal declarations shared by the libds4moe HIP sources.
//
// Library-owned device layout of one layer (all planes 256-byte aligned):
//
//   IQ2-style gate / up, per matrix [n_expert][n_ff rows][nbe = n_embd/256 blocks]:
//     qs plane  : 64 bytes per block = the 8 canonical sub-blocks of 8 bytes
//                 (4 codebook indices, then the sign/scale word), 8-byte aligned
//     d  plane  : fp16 d per block
//
//   Q2_K-style down, per matrix [n_expert][n_embd rows][nbf = n_ff/256 blocks]:
//     qs plane  : 64 bytes per block (canonical qs[64])
//     sc plane  : 16 bytes per block (canonical scales[16])
//     dd plane  : uint32 per block = d | dmin << 16 (fp16 bits)
//
// The planes hold exactly the canonical bytes (66 = 64 + 2, 84 = 64 + 16 + 4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ds4 {

constexpr int QK = 256;
constexpr int MAX_TOPK = 8;
constexpr int MAX_EXPERT = 256;
constexpr int GEMV_MAX_TOK = 4;   // GEMV path keeps up to this many tokens' x in registers

struct Layer {
    int n_embd, n_ff, n_expert, top_k, n_shared, max_tokens, act_dtype;
    int nbe, nbf;                   // blocks per gate/up row, per down row
    // weights (library-owned)
    const float *router;            // [NE][E]
    const float *router_bias;       // [NE] or nullptr
    const uint16_t *router_hml;     // [3][NE][E] bf16 parts hi, mid, lo of the router (hi + mid + lo = router)
    const float *router_norm;       // [NE] Euclidean norm of each router row, rounded up
    const uint16_t *codebook;       // [256] device copy
    const uint8_t *iq2_qs[2];       // gate, up: [NE][F][nbe][64]
    const uint16_t *iq2_d[2];       // [NE][F][nbe]
    const uint8_t *q2k_qs;          // [NE][E][nbf][64]
    const uint8_t *q2k_sc;          // [NE][E][nbf][16]
    const uint32_t *q2k_dd;         // [NE][E][nbf]
    const uint16_t *sh_gate, *sh_up, *sh_down;
};

// Workspace (device), carved from one allocation at create time.
struct Work {
    float *logits;        // [max_tokens][NE]
    int32_t *idx;         // [max_tokens][k]
    float *w;             // [max_tokens][k]
    int32_t *offsets;     // [NE+1]
    int32_t *list;        // [max_tokens*k] entries t*k + j, grouped by expert, ascending t
    int32_t *active;      // [NE+1]: active[0] = U, active[1..U] = experts with tokens, ascending
    int32_t *counters;    // counter slots of 256 bytes: slot 0 router tail, then the decode phases
    float *hbuf;          // [min(max_tokens, 4)*(k+1)][F] fp32 activations between gate/up and down (GEMV)
    // batched (GEMM) path
    uint16_t *hbuf16;     // [max_tokens*k][F] fp16 routed activations, row = slot t*k + j
    uint16_t *x16;        // [max_tokens][E] fp16 copy of x
    uint16_t *xhi, *xlo;  // [max_tokens][E] bf16 high / low parts of fp32 x (fp32 activations only)
    uint16_t *hsh_hi, *hsh_lo;  // [max_tokens][F] shared-expert activations, bf16 high / low parts
    float *part;          // [PART_ROWS][max(2F, E)] batched GEMMs: partial sums over K splits
    int4 *chunks;         // [gemm_max_chunks] (expert, first list position, count)
    int32_t *nchunks;     // number of valid chunks
    int32_t *ecount;      // [MAX_EXPERT] tokens per expert (batched router)
    float *rest;          // [4][max_tokens][NE] partial router estimates (batched router)
    unsigned long long *rtag;  // [MAX_EXPERT][2][2] fused decode: each fp64 half-row router
                               // sum as two 32-bit halves, each tagged with the call's epoch in its
                               // upper 32 bits
    unsigned long long *ltag;  // [64][MAX_EXPERT] small-batch router: fp32 logit bits under the call's tag
    unsigned long long *itag;  // [64][MAX_TOPK] small-batch router: selected expert under the call's tag
    unsigned long long *htag;  // [k+1][F] fused decode: SwiGLU outputs of the routed slots and the
                               // shared expert (fp32 bits), each tagged like rtag
};

// ---------------------------------------------------------------- small device helpers
// Weights are read once per call: non-temporal loads (streaming cache
// policy).  A plain streaming read with 512 workgroups of 256 threads and four
// 16-byte loads in flight per thread measured 7.2 TB/s with them on MI355X,
// 6.4 TB/s with ordinary loads.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt16(const void *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_nt4(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
}
__device__ __forceinline__ uint16_t ld_nt2(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(p));
}
__device__ __forceinline__ float4 ld_nt_f4(const float *p) {
    const uint4 v = ld_nt16(p);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float half_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// ---------------------------------------------------------------- host-side launchers
// Each returns hipGetLastError() after enqueueing.
hipError_t launch_repack_iq2(const uint8_t *canon, int64_t n_blocks, uint8_t *qs, uint16_t *d,
                             hipStream_t s);
hipError_t launch_repack_q2k(const uint8_t *canon, int64_t n_blocks, uint8_t *qs, uint8_t *sc,
                             uint32_t *dd, hipStream_t s);
hipError_t launch_dequant_iq2(const Layer &L, int which, int expert, float *dst, hipStream_t s);
hipError_t launch_dequant_q2k(const Layer &L, int expert, float *dst, hipStream_t s);

hipError_t launch_router_prep(const float *router, int NE, int E, uint16_t *hml, float *norm, hipStream_t s);
// ep: this handle's count of routing launches so far (the small-batch router's
// hand-off tag is ep + 1, never 0)
hipError_t launch_route(const Layer &L, const Work &W, const void *x, int n_tok, hipStream_t s,
                        unsigned long long ep);
hipError_t launch_route_export(const Layer &L, const Work &W, int n_tok, int32_t *idx, float *w,
                               int32_t *offsets, int32_t *tokens, hipStream_t s);

hipError_t launch_gemv_gateup_routed(const Layer &L, const Work &W, const void *x, int n_tok, hipStream_t s);
hipError_t launch_gemv_gateup_shared(const Layer &L, const Work &W, const void *x, int n_tok, hipStream_t s);
hipError_t launch_gemv_down_routed(const Layer &L, const Work &W, int n_tok, float *out, hipStream_t s);
hipError_t launch_gemv_down_shared(const Layer &L, const Work &W, int n_tok, float *out, hipStream_t s);

// Timing brackets recorded by ds4moe_forward when timing is enabled.
enum TimingKind {
    TK_ROUTE = 0, TK_GU_ROUTED = 1, TK_GU_SHARED = 2, TK_DN_ROUTED = 3, TK_DN_SHARED = 4,
    TK_GEMM_GU_ROUTED = 5, TK_GEMM_DN_ROUTED = 6, TK_FUSED = 7, TK_GEMM_PREP = 8, TK_GEMM_GU_SHARED = 9,
    TK_GEMM_DN_SHARED = 10, TK_COUNT = 11
};

bool gemm_enabled();
int gemm_max_chunks(int n_tok, int NE, int k);   // upper bound of the routed chunk count
constexpr int PART_ROWS = 2048;  // K splits times rows (tokens or slots) of a split GEMM launch, at most
hipError_t launch_gemm_prep(const Layer &L, const Work &W, const void *x, int n_tok, hipStream_t s);
hipError_t launch_gemm_gateup_routed(const Layer &L, const Work &W, int n_tok, hipStream_t s);
hipError_t launch_gemm_gateup_shared(const Layer &L, const Work &W, const void *x, int n_tok, hipStream_t s);
hipError_t launch_gemm_down_routed(const Layer &L, const Work &W, int n_tok, float *out, hipStream_t s);
hipError_t launch_gemm_down_shared(const Layer &L, const Work &W, int n_tok, float *out, hipStream_t s);

int decode_grid(int act_bf16);
hipError_t launch_decode_fused(const Layer &L, const Work &W, const void *x, float *out, int grid,
                               unsigned long long ep, hipStream_t s);

hipError_t launch_rmsnorm(const float *h, int n_tok, int n_embd, double eps, uint16_t *x, hipStream_t s);

}  // namespace ds4
