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
constexpr int SMALL_MAX_TOK = 8;  // small-batch kernels: tokens per call at most (bf16 x, 2-bit experts)
constexpr int SMALL_MAX_FF = 2048; // small-batch kernels: n_ff at most (h vectors staged in LDS)

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
    int fmt;                        // 0: IQ2 gate/up + Q2_K down; 1: Q4_K gate, up and down
    const uint8_t *q4_qs[3];        // Q4_K gate, up, down: [NE][rows][blocks][128] quants
    const uint4 *q4_meta[3];        //   and [NE][rows][blocks] 16-byte d | dmin | 6-bit fields
    // hash-routed layer: the experts of a token are row `id` of this table
    // ([n_vocab][top_k], library-owned), nullptr for a learned-routing layer
    const int32_t *hash_table;
    int n_vocab;
    // host-resident experts: the HBM slot holding each expert's weights
    // ([n_expert], set for the call by the cache update), nullptr when every
    // expert is resident in HBM (slot = expert)
    const int32_t *slot_of;
};

// The weight slot of expert e in the routed planes.
__device__ __forceinline__ int expert_slot(const Layer &L, int e) { return L.slot_of ? L.slot_of[e] : e; }

// HBM expert cache of a layer whose routed experts live in host memory
// (device memory, library-owned; every pointer a device address).
struct ExpertCache {
    int32_t *slot_of;       // [n_expert]: slot holding the expert, -1 if none
    int32_t *slot_expert;   // [slots]: expert held, -1 if empty
    uint32_t *slot_last;    // [slots]: cache clock of its last use (0 = never)
    uint32_t *clock;        // calls so far
    int32_t *miss_slot;     // [slots]: slots to fill in this call, in miss order
    int32_t *miss_count;
    unsigned long long *stats;  // calls, hits, misses, bytes loaded
    int slots;
};

// The routed planes of one expert, as (host-resident source, HBM slot base,
// bytes per expert): 7 planes for the 2-bit format, 6 for Q4_K.
struct ExpertPlanes {
    int n;
    const uint8_t *host[7];
    uint8_t *hbm[7];
    int64_t bytes[7];
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
    float *part2;         // the same for the shared expert's tiles when they run on a second stream (or null)
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
    // Bounded waits.  A wait that gives up stores its call's tag into *status,
    // a host-visible word (pinned host memory mapped into the device address
    // space), so the host sees the failure at its next call without
    // synchronising.  Consumers wait for (producer tag) ^ want_xor: 0 in normal
    // use; a nonzero value (set only by the test hook) makes every wait expire.
    uint32_t *status;
    int spin_limit;       // polls before a wait gives up
    uint32_t want_xor;
    // per call: the tokens' ids ([n_tok], device) for a hash-routed layer
    const int32_t *ids;
    // small-batch path: two buffers of gate/up sums in turn, each
    // [SMALL_MAX_TOK (k + 1)][2 F] fp32 (nullptr if the layer cannot take the path)
    float *sgu;
};

constexpr int DEFAULT_SPIN_LIMIT = 1 << 20;  // about a second of polling

// A bounded wait expired during the call tagged `tag`: record it for the host.
__device__ __forceinline__ void report_wait_expired(const Work &W, uint32_t tag) {
    __hip_atomic_store(W.status, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// A hash-routed call met a token id outside [0, n_vocab): record its tag in
// the status word's second slot.
__device__ __forceinline__ void report_bad_id(const Work &W, uint32_t tag) {
    __hip_atomic_store(W.status + 1, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ---------------------------------------------------------------- small device helpers
// Packed weights held across a loop over tokens: an empty asm that claims to
// change them keeps the compiler from hoisting their unpacking out of the
// loop (it would unpack every weight of the lane into registers, spill into
// AGPRs and wait for the loads before the first token).
__device__ __forceinline__ void keep_packed(uint4 &q) {
    asm volatile("" : "+v"(q.x), "+v"(q.y), "+v"(q.z), "+v"(q.w));
}
__device__ __forceinline__ void keep_packed(uint32_t &q) { asm volatile("" : "+v"(q)); }

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

// Wave-wide maximum of an unsigned key by DPP (row shifts, then the two row
// broadcasts), read from the last lane: every lane gets it.  All 64 lanes
// must be active.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true));  // row_shr:1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true));  // row_shr:2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true));  // row_shr:4
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true));  // row_shr:8
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false)); // row_bcast:15
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false)); // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Order-preserving 32-bit key of an fp32 logit (larger logit, larger key),
// never 0 (0 marks a taken or absent expert).
__device__ __forceinline__ uint32_t logit_key32(float L) {
    const uint32_t u = __float_as_uint(L);
    const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return key ? key : 1u;
}
__device__ __forceinline__ float key32_logit(uint32_t m) {
    return __uint_as_float((m & 0x80000000u) ? (m & 0x7FFFFFFFu) : ~m);
}

// One top-k round over the wave's keys (lane l holds experts l + 64 i in
// key[i]): the largest key, at the lowest expert index among equal keys; that
// expert's key is cleared.  Wave-uniform results.
__device__ __forceinline__ void topk_round(uint32_t (&key)[4], uint32_t &m, int &e) {
    const int lane = threadIdx.x & 63;
    m = wave_max_u32(max(max(key[0], key[1]), max(key[2], key[3])));
    e = -1;
#pragma unroll
    for (int i = 3; i >= 0; --i) {
        const uint64_t bb = __ballot(key[i] == m);
        if (bb) e = 64 * i + (__ffsll((unsigned long long)bb) - 1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (lane + 64 * i == e) key[i] = 0u;
}

// Sum and maximum over the wave's 64 lanes by DPP, in the tree of
// wave_max_u32 (prefixes within each 16-lane row, then the row broadcasts;
// lane 63 ends with the result, which every lane reads back), with no round
// trip through LDS: a shuffle tree costs one LDS permute per step and 32-bit
// half.  Lanes whose DPP source lies outside their row take the identity.
template <int CTRL, int ROW_MASK, bool BOUND>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, BOUND));
}
// Sum over each group of lpr consecutive lanes (lpr a power of two up to 64),
// left in the group's last lane, by DPP alone (row shifts, then the two row
// broadcasts): plain VALU work that never waits on LDS traffic in flight.
__device__ __forceinline__ float group_sum_last(float v, int lpr) {
    if (lpr > 1) v += dpp_f32<0x111, 0xF, true>(v);    // row_shr:1
    if (lpr > 2) v += dpp_f32<0x112, 0xF, true>(v);    // row_shr:2
    if (lpr > 4) v += dpp_f32<0x114, 0xF, true>(v);    // row_shr:4
    if (lpr > 8) v += dpp_f32<0x118, 0xF, true>(v);    // row_shr:8
    if (lpr > 16) v += dpp_f32<0x142, 0xA, false>(v);  // row_bcast:15
    if (lpr > 32) v += dpp_f32<0x143, 0xC, false>(v);  // row_bcast:31
    return v;
}
template <int CTRL, int ROW_MASK, bool BOUND>
__device__ __forceinline__ double dpp_f64(double v) {
    return __hiloint2double(__builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROW_MASK, 0xF, BOUND),
                            __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROW_MASK, 0xF, BOUND));
}
__device__ __forceinline__ double wave_sum_dpp(double v) {
    v += dpp_f64<0x111, 0xF, true>(v);   // row_shr:1
    v += dpp_f64<0x112, 0xF, true>(v);   // row_shr:2
    v += dpp_f64<0x114, 0xF, true>(v);   // row_shr:4
    v += dpp_f64<0x118, 0xF, true>(v);   // row_shr:8
    v += dpp_f64<0x142, 0xA, false>(v);  // row_bcast:15
    v += dpp_f64<0x143, 0xC, false>(v);  // row_bcast:31
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 63),
                            __builtin_amdgcn_readlane(__double2loint(v), 63));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max_f32(float v) {
    // a lane without a source keeps -inf (the old value; bound_ctrl off)
    const float o = __int_as_float(__builtin_amdgcn_update_dpp((int)0xFF800000u, __float_as_int(v), CTRL,
                                                               ROW_MASK, 0xF, false));
    return fmaxf(v, o);
}
__device__ __forceinline__ float wave_max_dpp(float v) {
    v = dpp_max_f32<0x111, 0xF>(v);
    v = dpp_max_f32<0x112, 0xF>(v);
    v = dpp_max_f32<0x114, 0xF>(v);
    v = dpp_max_f32<0x118, 0xF>(v);
    v = dpp_max_f32<0x142, 0xA>(v);
    v = dpp_max_f32<0x143, 0xC>(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_max_f64(double v) {
    // a lane without a source keeps -inf (0xFFF00000 00000000; bound_ctrl off)
    const double o = __hiloint2double(
        __builtin_amdgcn_update_dpp((int)0xFFF00000u, __double2hiint(v), CTRL, ROW_MASK, 0xF, false),
        __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROW_MASK, 0xF, false));
    return fmax(v, o);
}
__device__ __forceinline__ double wave_max_dpp(double v) {
    v = dpp_max_f64<0x111, 0xF>(v);
    v = dpp_max_f64<0x112, 0xF>(v);
    v = dpp_max_f64<0x114, 0xF>(v);
    v = dpp_max_f64<0x118, 0xF>(v);
    v = dpp_max_f64<0x142, 0xA>(v);
    v = dpp_max_f64<0x143, 0xC>(v);
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 63),
                            __builtin_amdgcn_readlane(__double2loint(v), 63));
}

// Lanes of the wave whose key equals this lane's (keys below 2^bits), by
// one ballot per key bit; every lane of the wave takes part.
__device__ __forceinline__ uint64_t wave_match_any(uint32_t key, int bits) {
    uint64_t m = ~0ull;
    for (int b = 0; b < bits; ++b) {
        const uint32_t kb = (key >> b) & 1u;
        const uint64_t bb = __ballot(kb);
        m &= kb ? bb : ~bb;
    }
    return m;
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
// hand-off tag is ep + 1, never 0).  lists = false: up to 64 tokens of a
// learned layer, the per-expert lists are not built (the small-batch kernels
// build them from W.idx); otherwise W holds the lists too.
hipError_t launch_route(const Layer &L, const Work &W, const void *x, int n_tok, hipStream_t s,
                        unsigned long long ep, bool lists = true);
// The shared expert of large bf16 calls on hipBLASLt (shared_blas.hip):
// gate/up GEMM + SiLU split into W.hsh_hi / hsh_lo, then the down GEMMs
// into out.  Requires sh_up == sh_gate + n_ff * n_embd.
struct SharedBlas;
constexpr int SBLAS_CHUNK = 2048;   // tokens per GEMM (the fp32 gate/up buffer holds one chunk)
constexpr int SBLAS_MIN_TOK = 128;  // calls of fewer tokens keep the grouped kernels' shared tiles
int sblas_create(SharedBlas **out, int n_ff);
void sblas_destroy(SharedBlas *S);
hipError_t sblas_gateup(SharedBlas *S, const Layer &L, const Work &W, const void *x, int n_tok, hipStream_t s);
hipError_t sblas_down(SharedBlas *S, const Layer &L, const Work &W, int n_tok, float *out, hipStream_t s);
hipError_t launch_debug_gemm_b(const Layer &L, int which, int expert, float *dst, hipStream_t s);
hipError_t launch_cache_update(const Layer &L, const Work &W, const ExpertCache &C, int64_t expert_bytes,
                               hipStream_t s);
hipError_t launch_cache_fill(const ExpertPlanes &P, const ExpertCache &C, hipStream_t s);
hipError_t launch_fill_u32(uint32_t *p, int n, uint32_t v, hipStream_t s);
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
    TK_GEMM_DN_SHARED = 10, TK_Q4_GU_ROUTED = 11, TK_Q4_DN_ROUTED = 12, TK_CACHE = 13, TK_SMALL_GU = 14,
    TK_SMALL_DN = 15, TK_COUNT = 16
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
// pre_routed: the routing of the token is already in W (the router kernel ran
// earlier on the stream), so the kernel skips its router phase.
hipError_t launch_decode_fused(const Layer &L, const Work &W, const void *x, float *out, int grid,
                               unsigned long long ep, hipStream_t s, bool pre_routed = false);

// Small batches (2..SMALL_MAX_TOK tokens, bf16 x, 2-bit experts), after the
// router: gate/up sums into gu (small_sum_floats floats, zero on entry), then
// the down projections into out, which also clear gz (the other buffer).
int small_grid();  // workgroups per launch (one per CU), 0 if the kernels cannot run
size_t small_sum_floats(const Layer &L);
hipError_t launch_small_gateup(const Layer &L, const Work &W, const void *x, int n_tok, float *gu, int grid,
                               hipStream_t s);
hipError_t launch_small_down(const Layer &L, const Work &W, const float *gu, float *gz, int n_tok, float *out,
                             int grid, hipStream_t s);

hipError_t launch_rmsnorm(const float *h, int n_tok, int n_embd, double eps, uint16_t *x, hipStream_t s);

hipError_t launch_repack_q4k(const uint8_t *canon, int64_t n_blocks, uint4 *meta, uint8_t *qs, hipStream_t s);
hipError_t launch_dequant_q4k(const Layer &L, int which, int expert, float *dst, hipStream_t s);
hipError_t launch_q4_gateup_routed(const Layer &L, const Work &W, const void *x, int n_tok, hipStream_t s);
hipError_t launch_q4_down_routed(const Layer &L, const Work &W, int n_tok, float *out, hipStream_t s);

}  // namespace ds4
