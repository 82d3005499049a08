// cache.hip - HBM expert cache for routed experts that live in host memory.
//
// When the model does not fit in the GPU's memory, the pages keep the
// non-routed weights (shared expert, projections) resident and load a routed
// expert from the model file when a token needs one that is not resident,
// releasing cache space for it ("DS-4 DwarfStar - DeepSeek V4 Flash 本地推理引擎",
// section "SSD Streaming", how it works; "ds4 深度实战...", section 3.5).
// Here the backing store is pinned host memory holding the routed experts in
// the library's own plane layout, and HBM holds a fixed number of expert
// slots; the least recently used expert leaves first.  Everything runs on the
// call's stream after the router, with no host round trip:
//   k_cache_update (one workgroup): marks this call's resident experts as used
//     now, lists the missing ones in ascending expert order, picks as many
//     victim slots among the slots this call does not use (empty ones first,
//     then least recently used, lower slot first on equal stamps), moves the
//     expert -> slot map and counts hits, misses and bytes;
//   k_cache_fill: copies each missed expert's planes from host memory into
//     its slot over the host link (16-byte loads, many in flight);
// and the expert kernels then read expert e's weights at slot slot_of[e].
#include "common.h"

namespace ds4 {

// n_expert <= 256 and slots <= 256: one thread per expert and per slot.
__global__ __launch_bounds__(256) void k_cache_update(Work W, ExpertCache C, int64_t expert_bytes) {
    __shared__ uint32_t last[MAX_EXPERT];
    __shared__ int miss_e[MAX_EXPERT];
    __shared__ int victim[MAX_EXPERT];
    __shared__ int wmiss[4];
    __shared__ uint32_t now;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int S = C.slots;
    const int U = W.active[0];
    if (tid == 0) {
        now = *C.clock + 1u;
        *C.clock = now;
    }
    if (tid < S) last[tid] = C.slot_last[tid];
    victim[tid] = 0;  // stays in bounds even if a call had more misses than free slots
    __syncthreads();
    // this call's experts (ascending): hits are stamped now, misses flagged
    int e = -1;
    bool miss = false;
    if (tid < U) {
        e = W.active[1 + tid];
        const int s = C.slot_of[e];
        if (s >= 0)
            last[s] = now;
        else
            miss = true;
    }
    // misses in ascending expert order (a scan over the four waves)
    const uint64_t bm = __ballot(miss);
    if (lane == 0) wmiss[wave] = __popcll(bm);
    __syncthreads();
    int pre = 0;
    for (int w = 0; w < wave; ++w) pre += wmiss[w];
    const int M = wmiss[0] + wmiss[1] + wmiss[2] + wmiss[3];
    if (miss) miss_e[pre + __popcll(bm & ((1ull << lane) - 1ull))] = e;
    // victims: the slots this call does not use, ordered by (stamp, slot)
    if (tid < S && last[tid] != now) {
        const uint32_t mine = last[tid];
        int rank = 0;
        for (int s = 0; s < S; ++s) {
            const uint32_t o = last[s];
            rank += (o != now) && (o < mine || (o == mine && s < tid));
        }
        if (rank < M) victim[rank] = tid;
    }
    __syncthreads();
    // Every miss gets a victim: the host splits a call so that its distinct
    // experts fit in the slots (n_tok * top_k <= slots, or n_expert <= slots).
    if (tid < M) {
        const int s = victim[tid];
        const int ne = miss_e[tid];
        const int old = C.slot_expert[s];
        if (old >= 0) C.slot_of[old] = -1;  // an expert this call does not use
        C.slot_of[ne] = s;
        C.slot_expert[s] = ne;
        last[s] = now;
        C.miss_slot[tid] = s;
    }
    __syncthreads();
    if (tid < S) C.slot_last[tid] = last[tid];
    if (tid == 0) {
        *C.miss_count = M;
        C.stats[0] += 1ull;
        C.stats[1] += (unsigned long long)(U - M);
        C.stats[2] += (unsigned long long)M;
        C.stats[3] += (unsigned long long)M * (unsigned long long)expert_bytes;
    }
}

// Copy the missed experts' planes, host -> HBM slot.  The 16-byte units of
// one expert are numbered over its planes in order; each thread moves 4 units
// per step, all 4 loads issued before the stores.
constexpr int CF_UNROLL = 4;
__global__ __launch_bounds__(256) void k_cache_fill(ExpertPlanes P, ExpertCache C) {
    const int M = *C.miss_count;
    if (M == 0) return;
    int64_t per = 0;
    for (int i = 0; i < P.n; ++i) per += P.bytes[i] >> 4;
    const int64_t total = (int64_t)M * per;
    const int64_t stride = (int64_t)gridDim.x * 256 * CF_UNROLL;
    for (int64_t u0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * CF_UNROLL; u0 < total; u0 += stride) {
        uint4 v[CF_UNROLL];
        uint4 *dst[CF_UNROLL];
#pragma unroll
        for (int j = 0; j < CF_UNROLL; ++j) {
            dst[j] = nullptr;
            const int64_t u = u0 + j;
            if (u < total) {
                const int m = (int)(u / per);
                int64_t r = u - (int64_t)m * per;
                int seg = 0;
                while (r >= (P.bytes[seg] >> 4)) r -= P.bytes[seg] >> 4, ++seg;
                const int s = C.miss_slot[m];
                const int e = C.slot_expert[s];
                v[j] = *reinterpret_cast<const uint4 *>(P.host[seg] + (int64_t)e * P.bytes[seg] + 16 * r);
                dst[j] = reinterpret_cast<uint4 *>(P.hbm[seg] + (int64_t)s * P.bytes[seg] + 16 * r);
            }
        }
#pragma unroll
        for (int j = 0; j < CF_UNROLL; ++j)
            if (dst[j]) *dst[j] = v[j];
    }
}

hipError_t launch_cache_update(const Layer &L, const Work &W, const ExpertCache &C, int64_t expert_bytes,
                               hipStream_t s) {
    (void)L;
    hipLaunchKernelGGL(k_cache_update, dim3(1), dim3(256), 0, s, W, C, expert_bytes);
    return hipGetLastError();
}

hipError_t launch_cache_fill(const ExpertPlanes &P, const ExpertCache &C, hipStream_t s) {
    hipLaunchKernelGGL(k_cache_fill, dim3(1024), dim3(256), 0, s, P, C);
    return hipGetLastError();
}

}  // namespace ds4
