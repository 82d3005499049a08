// ds4moe.hip - host side of libds4moe.so: the C ABI declared in include/ds4moe.h.
//
// create() owns every device buffer of a layer (repacked experts, router and
// shared-expert copies, workspace); route()/forward() only validate and enqueue
// kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "ds4moe.h"
#include "common.h"

using namespace ds4;

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

bool pow2_dim(int v) { return v == 256 || v == 512 || v == 1024 || v == 2048 || v == 4096; }

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

constexpr int TIMING_SLOTS = TK_COUNT;
static_assert(TIMING_SLOTS == DS4MOE_TIMING_KINDS, "timing kinds of the ABI");
constexpr int TIMING_EVENTS = 4096;

// ---------------------------------------------------------------- static scratch
// The scratch of ds4moe_forward_static: one array per GPU, in device memory
// the library never allocates (the code object's own storage), holding the
// routing results, the tagged hand-off words, the router's tickets and the
// SwiGLU activations of calls of 1..4 tokens.  In host code its name is only a
// stand-in: kernels get the address that hipGetSymbolAddress returned for the
// device, looked up once per device with that device current.
constexpr size_t STATIC_BYTES = DS4MOE_STATIC_SCRATCH_BYTES;
constexpr int STATIC_MAX_TOK = DS4MOE_STATIC_MAX_TOKENS;
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES] = {};
// Calls on a device's array: their hand-off tags, unique across the handles
// that share it.
std::atomic<unsigned long long> g_static_calls[MAX_DEVICES];

}  // namespace

static __device__ __align__(256) unsigned char scratch[STATIC_BYTES];

struct ds4moe {
    Layer L{};
    Work W{};
    int path = DS4MOE_PATH_AUTO;
    int decode_grid = 0;    // workgroups of the persistent decode kernel
    int small_grid = 0;     // workgroups of the small-batch kernels (0: the layer has no small-batch path)
    int small_parity = 0;   // which of the two gate/up sum buffers the next small-batch call uses
    unsigned long long decode_calls = 0;  // fused launches so far (the phase counters' epoch)
    unsigned long long route_calls = 0;   // routing launches so far (the router hand-off tag)
    bool poisoned = false;
    std::string poison_why;               // what poisoned it, repeated by every later call
    int device = 0;
    int32_t last_n_tok = -1;              // n_tok of the latest forward/route call (its routing is in W)
    bool last_static = false;             // ... made by ds4moe_forward_static (its routing is in Wst)
    Work Wst{};                           // the workspace of ds4moe_forward_static, in the static scratch
    size_t static_need = 0;               // bytes of it this layer needs
    uint32_t *status_host = nullptr;      // pinned, mapped: nonzero = a bounded wait expired (that call's tag)
    std::vector<void *> allocs;
    // host-resident experts (cache.slots > 0): the HBM cache, the planes it
    // copies, and the layer as seen from the host store (for dequantize)
    ExpertCache cache{};
    ExpertPlanes planes{};
    int64_t expert_bytes = 0;
    Layer Lhost{};
    std::vector<void *> host_allocs;      // pinned host memory of the backing store
    SharedBlas *sblas = nullptr;          // the shared expert of large bf16 calls on hipBLASLt, if any
    // a stream for the shared expert of calls on the grouped path (bf16
    // tokens), which then runs beside the routing and the routed gate/up GEMM
    // (forked from and joined back into the caller's stream within the call)
    hipStream_t s2 = nullptr;
    hipEvent_t ev_fork = nullptr, ev_join = nullptr;
    // timing
    bool timing = false;
    std::vector<hipEvent_t> events;  // pairs
    std::vector<int> event_kind;
    int n_events = 0;
    double ms[TIMING_SLOTS] = {};
    int64_t counts[TIMING_SLOTS] = {};

    ~ds4moe() {
        for (void *p : allocs) (void)hipFree(p);
        for (hipEvent_t e : events) (void)hipEventDestroy(e);
        if (status_host) (void)hipHostFree(status_host);
        for (void *p : host_allocs) (void)hipHostFree(p);
        sblas_destroy(sblas);
        if (ev_fork) (void)hipEventDestroy(ev_fork);
        if (ev_join) (void)hipEventDestroy(ev_join);
        if (s2) (void)hipStreamDestroy(s2);
    }
    void *alloc(size_t bytes, hipError_t &err) {
        void *p = nullptr;
        err = hipMalloc(&p, align256(bytes ? bytes : 1));
        if (err == hipSuccess) allocs.push_back(p);
        return p;
    }
    // Timing brackets: begin/end around a kernel group.
    int tbegin(int kind, hipStream_t s) {
        if (!timing || n_events + 2 > (int)events.size()) return -1;
        int i = n_events;
        n_events += 2;
        event_kind[i / 2] = kind;
        hipEventRecord(events[i], s);
        return i;
    }
    void tend(int i, hipStream_t s) {
        if (i >= 0) hipEventRecord(events[i + 1], s);
    }
};

static bool gemm_available() { return ds4::gemm_enabled(); }

static int check_launch(ds4moe *h, hipError_t e, const char *what) {
    if (e != hipSuccess) {
        h->poisoned = true;
        h->poison_why = std::string(what) + ": " + hipGetErrorString(e);
        return fail(DS4MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
    }
    return DS4MOE_OK;
}

// Carve the forward_static workspace (1..4 tokens: the fused decode and the
// GEMV path) out of the device's static scratch; returns the bytes it spans.
static size_t carve_static(const Layer &L, char *base, Work &S) {
    const size_t T = STATIC_MAX_TOK, NE = L.n_expert, k = L.top_k, F = L.n_ff;
    size_t off = 0;
    auto carve = [&](size_t bytes) { char *p = base + off; off += align256(bytes); return p; };
    S.idx = (int32_t *)carve(T * k * 4);
    S.w = (float *)carve(T * k * 4);
    S.offsets = (int32_t *)carve((NE + 1) * 4);
    S.list = (int32_t *)carve(T * k * 4);
    S.active = (int32_t *)carve((NE + 1) * 4);
    S.counters = (int32_t *)carve(256);
    S.rtag = (unsigned long long *)carve(4 * MAX_EXPERT * 8);
    S.htag = (unsigned long long *)carve((k + 1) * F * 8);
    S.ltag = (unsigned long long *)carve(T * MAX_EXPERT * 8);
    S.itag = (unsigned long long *)carve(T * MAX_TOPK * 8);
    S.hbuf = (float *)carve(T * (k + 1) * F * 4);
    return off;
}

// The expert kernels of a q4 layer after the routing, for at most
// GEMV_MAX_TOK tokens: shared gate/up, routed gate/up (Q4_K), routed down
// (Q4_K), shared down.
static int run_q4_experts(ds4moe *h, const Work &W, const void *x, int n, float *out, hipStream_t s, bool timed) {
    const Layer &L = h->L;
    int tb, rc = DS4MOE_OK;
    if (L.n_shared) {
        tb = timed ? h->tbegin(TK_GU_SHARED, s) : -1;
        rc = check_launch(h, launch_gemv_gateup_shared(L, W, x, n, s), "q4 shared gate/up");
        h->tend(tb, s);
        if (rc) return rc;
    }
    tb = timed ? h->tbegin(TK_Q4_GU_ROUTED, s) : -1;
    rc = check_launch(h, launch_q4_gateup_routed(L, W, x, n, s), "q4 routed gate/up");
    h->tend(tb, s);
    if (rc) return rc;
    tb = timed ? h->tbegin(TK_Q4_DN_ROUTED, s) : -1;
    rc = check_launch(h, launch_q4_down_routed(L, W, n, out, s), "q4 routed down");
    h->tend(tb, s);
    if (rc) return rc;
    if (L.n_shared) {
        tb = timed ? h->tbegin(TK_DN_SHARED, s) : -1;
        rc = check_launch(h, launch_gemv_down_shared(L, W, n, out, s), "q4 shared down");
        h->tend(tb, s);
    }
    return rc;
}

// One call of at most GEMV_MAX_TOK tokens on a q4 layer: router, then the
// expert kernels.
static int run_q4_chunk(ds4moe *h, const Work &W, const void *x, int n, float *out, unsigned long long ep,
                        hipStream_t s, bool timed) {
    int tb = timed ? h->tbegin(TK_ROUTE, s) : -1;
    int rc = check_launch(h, launch_route(h->L, W, x, n, s, ep), "q4 route");
    h->tend(tb, s);
    if (rc) return rc;
    return run_q4_experts(h, W, x, n, out, s, timed);
}

extern "C" {

const char *ds4moe_last_error(void) { return g_err.c_str(); }

int ds4moe_create(const ds4moe_desc *d, void *stream, ds4moe_t **out) {
    if (!d || !out) return fail(DS4MOE_EINVAL, "create: NULL desc or out");
    if (d->abi_version != DS4MOE_ABI_VERSION)
        return fail(DS4MOE_EINVAL, "create: abi_version %d, library is %d", d->abi_version, DS4MOE_ABI_VERSION);
    if (!pow2_dim(d->n_embd) || !pow2_dim(d->n_ff))
        return fail(DS4MOE_EINVAL, "create: n_embd %d / n_ff %d must be one of 256..4096 (powers of two)",
                    d->n_embd, d->n_ff);
    if (d->n_expert < 1 || d->n_expert > MAX_EXPERT)
        return fail(DS4MOE_EINVAL, "create: n_expert %d not in 1..%d", d->n_expert, MAX_EXPERT);
    if (d->top_k < 1 || d->top_k > MAX_TOPK || d->top_k > d->n_expert)
        return fail(DS4MOE_EINVAL, "create: top_k %d not in 1..min(n_expert, %d)", d->top_k, MAX_TOPK);
    if (d->n_shared != 0 && d->n_shared != 1) return fail(DS4MOE_EINVAL, "create: n_shared must be 0 or 1");
    if (d->max_tokens < 1 || d->max_tokens > (1 << 20))
        return fail(DS4MOE_EINVAL, "create: max_tokens %d not in 1..2^20", d->max_tokens);
    if (d->act_dtype != DS4MOE_F32 && d->act_dtype != DS4MOE_BF16)
        return fail(DS4MOE_EINVAL, "create: act_dtype %d", d->act_dtype);
    if (d->expert_format != DS4MOE_FMT_Q2 && d->expert_format != DS4MOE_FMT_Q4)
        return fail(DS4MOE_EINVAL, "create: expert_format %d", d->expert_format);
    const bool q4 = d->expert_format == DS4MOE_FMT_Q4;
    if (!d->router || !d->gate || !d->up || !d->down || (!q4 && !d->codebook))
        return fail(DS4MOE_EINVAL, "create: NULL router/gate/up/down/codebook");
    if (d->n_shared && (!d->sh_gate || !d->sh_up || !d->sh_down))
        return fail(DS4MOE_EINVAL, "create: n_shared = 1 but a shared-expert pointer is NULL");
    if (d->expert_cache_slots < 0 || d->expert_cache_slots > d->n_expert ||
        (d->expert_cache_slots > 0 && d->expert_cache_slots < d->top_k))
        return fail(DS4MOE_EINVAL, "create: expert_cache_slots %d not 0 or in top_k..n_expert (%d..%d)",
                    d->expert_cache_slots, d->top_k, d->n_expert);
    if (d->hash_table) {
        if (d->n_vocab < 1 || d->n_vocab > (int64_t)(INT32_MAX / d->top_k))
            return fail(DS4MOE_EINVAL, "create: n_vocab %lld for a hash table", (long long)d->n_vocab);
        if ((uintptr_t)d->hash_table & 3u) return fail(DS4MOE_EINVAL, "create: hash_table is not 4-byte aligned");
    }

    hipStream_t s = (hipStream_t)stream;
    ds4moe *h = new (std::nothrow) ds4moe();
    if (!h) return fail(DS4MOE_ENOMEM, "create: host allocation");
    hipGetDevice(&h->device);
    Layer &L = h->L;
    L.n_embd = d->n_embd, L.n_ff = d->n_ff, L.n_expert = d->n_expert, L.top_k = d->top_k;
    L.n_shared = d->n_shared, L.max_tokens = d->max_tokens, L.act_dtype = d->act_dtype;
    L.nbe = d->n_embd / QK, L.nbf = d->n_ff / QK;
    const int64_t E = d->n_embd, F = d->n_ff, NE = d->n_expert, k = d->top_k, T = d->max_tokens;
    const int64_t gu_blocks = NE * F * L.nbe, dn_blocks = NE * E * L.nbf;

    hipError_t err = hipSuccess;
    auto A = [&](size_t bytes) -> void * {
        if (err != hipSuccess) return nullptr;
        return h->alloc(bytes, err);
    };
    float *router = (float *)A(NE * E * 4);
    float *bias = d->router_bias ? (float *)A(NE * 4) : nullptr;
    uint16_t *rhml = (uint16_t *)A(3 * NE * E * 2);
    float *rnorm = (float *)A(NE * 4);
    uint16_t *cb = (uint16_t *)A(512);
    const int64_t n_hash = d->hash_table ? d->n_vocab * k : 0;
    int32_t *htab = d->hash_table ? (int32_t *)A(n_hash * 4) : nullptr;
    // the routed planes of the layer's format (the other format's stay NULL)
    uint8_t *gq = nullptr, *uq = nullptr, *dq = nullptr, *dsc = nullptr;
    uint16_t *gd = nullptr, *ud = nullptr;
    uint32_t *ddd = nullptr;
    uint8_t *q4q[3] = {nullptr, nullptr, nullptr};
    uint4 *q4m[3] = {nullptr, nullptr, nullptr};
    // HBM holds the planes of every expert, or of `slots` experts when the
    // routed experts live in host memory (their planes are then in pinned host
    // memory, for all experts, in the same layout)
    const int S = d->expert_cache_slots;
    const int64_t NR = S ? S : NE;
    const int64_t gu_pe = F * L.nbe, dn_pe = E * L.nbf;  // blocks per expert
    if (q4) {
        const int64_t nbk[3] = {gu_pe * NR, gu_pe * NR, dn_pe * NR};
        for (int i = 0; i < 3; ++i) q4q[i] = (uint8_t *)A(nbk[i] * 128), q4m[i] = (uint4 *)A(nbk[i] * 16);
    } else {
        gq = (uint8_t *)A(gu_pe * NR * 64), uq = (uint8_t *)A(gu_pe * NR * 64);
        gd = (uint16_t *)A(gu_pe * NR * 2), ud = (uint16_t *)A(gu_pe * NR * 2);
        dq = (uint8_t *)A(dn_pe * NR * 64), dsc = (uint8_t *)A(dn_pe * NR * 16);
        ddd = (uint32_t *)A(dn_pe * NR * 4);
    }
    // pinned host store and cache state
    bool host_ok = true;
    auto H = [&](size_t bytes) -> uint8_t * {
        void *p = nullptr, *dp = nullptr;
        if (!host_ok || hipHostMalloc(&p, align256(bytes), hipHostMallocMapped) != hipSuccess) {
            host_ok = false;
            return nullptr;
        }
        h->host_allocs.push_back(p);
        if (hipHostGetDevicePointer(&dp, p, 0) != hipSuccess) host_ok = false;
        return (uint8_t *)dp;
    };
    uint8_t *hgq = nullptr, *huq = nullptr, *hgd = nullptr, *hud = nullptr, *hdq = nullptr, *hdsc = nullptr,
            *hddd = nullptr, *hq4q[3] = {nullptr, nullptr, nullptr}, *hq4m[3] = {nullptr, nullptr, nullptr};
    int32_t *cstate = nullptr;
    if (S) {
        if (q4) {
            const int64_t nbk[3] = {gu_blocks, gu_blocks, dn_blocks};
            for (int i = 0; i < 3; ++i) hq4q[i] = H(nbk[i] * 128), hq4m[i] = H(nbk[i] * 16);
        } else {
            hgq = H(gu_blocks * 64), huq = H(gu_blocks * 64), hgd = H(gu_blocks * 2), hud = H(gu_blocks * 2);
            hdq = H(dn_blocks * 64), hdsc = H(dn_blocks * 16), hddd = H(dn_blocks * 4);
        }
        // slot_of [NE], slot_expert [S], slot_last [S], miss_slot [S], clock, miss_count, stats [4]
        cstate = (int32_t *)A((NE + 3 * S + 2) * 4 + 64);
    }
    uint16_t *sg = nullptr, *su = nullptr, *sd = nullptr;
    if (d->n_shared) {
        // gate and up adjacent: one [2 n_ff][n_embd] matrix for the library GEMM
        sg = (uint16_t *)A(2 * F * E * 2);
        su = sg ? sg + F * E : nullptr;
        sd = (uint16_t *)A(E * F * 2);
    }
    // workspace
    const int64_t gemv_slots = std::min<int64_t>(T, GEMV_MAX_TOK) * (k + 1);
    size_t off = 0;
    auto carve = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    size_t o_logits = carve(T * NE * 4), o_idx = carve(T * k * 4), o_w = carve(T * k * 4);
    size_t o_off = carve((NE + 1) * 4), o_list = carve(T * k * 4), o_act = carve((NE + 1) * 4);
    size_t o_cnt = carve(16 * 256), o_h = carve(gemv_slots * F * 4), o_h16 = carve(T * k * F * 2);
    size_t o_x16 = carve(T * E * 2);
    const bool xf32 = d->act_dtype == DS4MOE_F32;
    size_t o_xhi = carve(xf32 ? T * E * 2 : 0), o_xlo = carve(xf32 ? T * E * 2 : 0);
    size_t o_shh = carve(d->n_shared ? T * F * 2 : 0), o_shl = carve(d->n_shared ? T * F * 2 : 0);
    size_t o_part = carve((size_t)PART_ROWS * std::max<int64_t>(2 * F, E) * 4);
    // a second one for the shared expert's tiles, which run beside the routed
    // GEMMs on a second stream in calls of bf16 tokens on the grouped path
    const bool fork_tiles = !xf32 && d->n_shared && T >= 2;
    size_t o_part2 = carve(fork_tiles ? (size_t)PART_ROWS * std::max<int64_t>(2 * F, E) * 4 : 0);
    size_t o_chunks = carve((size_t)gemm_max_chunks((int)T, (int)NE, (int)k) * 16), o_nch = carve(4);
    size_t o_ecnt = carve(MAX_EXPERT * 4), o_rest = carve(4 * T * NE * 4), o_rtag = carve(4 * MAX_EXPERT * 8);
    size_t o_htag = carve((size_t)(k + 1) * F * 8);
    size_t o_ltag = carve(64 * MAX_EXPERT * 8), o_itag = carve(64 * MAX_TOPK * 8);
    // small batches (2..SMALL_MAX_TOK bf16 tokens, 2-bit experts, n_ff <= SMALL_MAX_FF): two
    // gate/up sum buffers, zero at create like the whole workspace
    const bool small_cap = !q4 && d->act_dtype == DS4MOE_BF16 && T >= 2 && F <= SMALL_MAX_FF;
    size_t o_sgu = carve(small_cap ? 2 * small_sum_floats(L) * 4 : 0);
    char *ws = (char *)A(off);
    if (err != hipSuccess) {
        delete h;
        hipGetLastError();
        return fail(DS4MOE_ENOMEM, "create: device allocation failed (%s)", hipGetErrorString(err));
    }
    if (!host_ok) {
        delete h;
        hipGetLastError();
        return fail(DS4MOE_ENOMEM, "create: pinned host memory for the host-resident experts");
    }
    if (S) {
        ExpertCache &C = h->cache;
        C.slots = S;
        C.slot_of = cstate;
        C.slot_expert = cstate + NE;
        C.slot_last = (uint32_t *)(cstate + NE + S);
        C.miss_slot = cstate + NE + 2 * S;
        C.clock = (uint32_t *)(cstate + NE + 3 * S);
        C.miss_count = cstate + NE + 3 * S + 1;
        // 8-byte aligned, within the 64 bytes allocated past the counters
        C.stats = (unsigned long long *)(((uintptr_t)(cstate + NE + 3 * S + 2) + 7) & ~(uintptr_t)7);
    }
    Work &W = h->W;
    W.logits = (float *)(ws + o_logits);
    W.idx = (int32_t *)(ws + o_idx);
    W.w = (float *)(ws + o_w);
    W.offsets = (int32_t *)(ws + o_off);
    W.list = (int32_t *)(ws + o_list);
    W.active = (int32_t *)(ws + o_act);
    W.counters = (int32_t *)(ws + o_cnt);
    W.hbuf = (float *)(ws + o_h);
    W.hbuf16 = (uint16_t *)(ws + o_h16);
    W.x16 = (uint16_t *)(ws + o_x16);
    W.xhi = xf32 ? (uint16_t *)(ws + o_xhi) : nullptr;
    W.xlo = xf32 ? (uint16_t *)(ws + o_xlo) : nullptr;
    W.hsh_hi = d->n_shared ? (uint16_t *)(ws + o_shh) : nullptr;
    W.hsh_lo = d->n_shared ? (uint16_t *)(ws + o_shl) : nullptr;
    W.part = (float *)(ws + o_part);
    W.part2 = fork_tiles ? (float *)(ws + o_part2) : nullptr;
    W.chunks = (int4 *)(ws + o_chunks);
    W.nchunks = (int32_t *)(ws + o_nch);
    W.ecount = (int32_t *)(ws + o_ecnt);
    W.rest = (float *)(ws + o_rest);
    W.rtag = (unsigned long long *)(ws + o_rtag);
    W.htag = (unsigned long long *)(ws + o_htag);
    W.ltag = (unsigned long long *)(ws + o_ltag);
    W.itag = (unsigned long long *)(ws + o_itag);
    W.sgu = small_cap ? (float *)(ws + o_sgu) : nullptr;
    // the host-visible status word of the bounded waits
    if (hipHostMalloc((void **)&h->status_host, 256, hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess) {
        h->status_host = nullptr;
        delete h;
        hipGetLastError();
        return fail(DS4MOE_ENOMEM, "create: pinned status word");
    }
    ((volatile uint32_t *)h->status_host)[0] = 0u;  // a bounded wait expired (that call's tag)
    ((volatile uint32_t *)h->status_host)[1] = 0u;  // a token id out of range (that call's tag)
    if (hipHostGetDevicePointer((void **)&W.status, h->status_host, 0) != hipSuccess) {
        delete h;
        hipGetLastError();
        return fail(DS4MOE_EHIP, "create: device address of the status word");
    }
    W.spin_limit = DEFAULT_SPIN_LIMIT;
    W.want_xor = 0u;
    // the device's static scratch (ds4moe_forward_static): its address, looked
    // up once per device with the device current
    if (h->device < 0 || h->device >= MAX_DEVICES) {
        delete h;
        return fail(DS4MOE_EUNSUPPORTED, "create: device %d beyond the library's table", h->device);
    }
    {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        if (!g_scratch_ptr[h->device]) {
            void *p = nullptr;
            hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p) {
                delete h;
                hipGetLastError();
                return fail(DS4MOE_EHIP, "create: address of the static scratch (%s)", hipGetErrorString(e));
            }
            g_scratch_ptr[h->device] = p;
        }
        h->Wst = Work{};
        h->Wst.status = W.status;
        h->static_need = carve_static(L, (char *)g_scratch_ptr[h->device], h->Wst);
    }

#define CK(call)                                                                                      \
    do {                                                                                              \
        hipError_t e_ = (call);                                                                       \
        if (e_ != hipSuccess) {                                                                       \
            delete h;                                                                                 \
            return fail(DS4MOE_EHIP, "create: %s: %s", #call, hipGetErrorString(e_));                 \
        }                                                                                             \
    } while (0)
    CK(hipMemsetAsync(ws, 0, off, s));
    std::vector<int32_t> host_table;
    if (htab) {
        host_table.resize((size_t)n_hash);
        CK(hipMemcpyAsync(htab, d->hash_table, n_hash * 4, hipMemcpyDeviceToDevice, s));
        CK(hipMemcpyAsync(host_table.data(), d->hash_table, n_hash * 4, hipMemcpyDeviceToHost, s));
    }
    CK(hipMemcpyAsync(router, d->router, NE * E * 4, hipMemcpyDeviceToDevice, s));
    if (bias) CK(hipMemcpyAsync(bias, d->router_bias, NE * 4, hipMemcpyDeviceToDevice, s));
    CK(launch_router_prep(router, (int)NE, (int)E, rhml, rnorm, s));
    if (!q4) CK(hipMemcpyAsync(cb, d->codebook, 512, hipMemcpyHostToDevice, s));
    if (d->n_shared) {
        CK(hipMemcpyAsync(sg, d->sh_gate, F * E * 2, hipMemcpyDeviceToDevice, s));
        CK(hipMemcpyAsync(su, d->sh_up, F * E * 2, hipMemcpyDeviceToDevice, s));
        CK(hipMemcpyAsync(sd, d->sh_down, E * F * 2, hipMemcpyDeviceToDevice, s));
    }
    if (S) {
        // empty cache: no expert resident (-1), stamps, clock, counters 0
        CK(hipMemsetAsync(cstate, 0xFF, (NE + S) * 4, s));
        CK(hipMemsetAsync(cstate + NE + S, 0, (2 * S + 2) * 4 + 64, s));
    }
    // the repacked planes go to HBM, or to the host store (all experts)
    if (q4) {
        if (((uintptr_t)d->gate | (uintptr_t)d->up | (uintptr_t)d->down) & 15u) {
            delete h;
            return fail(DS4MOE_EINVAL, "create: Q4_K weights must be 16-byte aligned");
        }
        uint8_t *tq[3], *tm[3];
        for (int i = 0; i < 3; ++i) tq[i] = S ? hq4q[i] : q4q[i], tm[i] = S ? hq4m[i] : (uint8_t *)q4m[i];
        CK(launch_repack_q4k((const uint8_t *)d->gate, gu_blocks, (uint4 *)tm[0], tq[0], s));
        CK(launch_repack_q4k((const uint8_t *)d->up, gu_blocks, (uint4 *)tm[1], tq[1], s));
        CK(launch_repack_q4k((const uint8_t *)d->down, dn_blocks, (uint4 *)tm[2], tq[2], s));
    } else {
        CK(launch_repack_iq2((const uint8_t *)d->gate, gu_blocks, S ? hgq : gq, S ? (uint16_t *)hgd : gd, s));
        CK(launch_repack_iq2((const uint8_t *)d->up, gu_blocks, S ? huq : uq, S ? (uint16_t *)hud : ud, s));
        CK(launch_repack_q2k((const uint8_t *)d->down, dn_blocks, S ? hdq : dq, S ? hdsc : dsc,
                             S ? (uint32_t *)hddd : ddd, s));
    }
    CK(hipStreamSynchronize(s));
#undef CK
    // every table row: k distinct experts in range (the kernels index with them unchecked)
    for (int64_t v = 0; v < (int64_t)host_table.size() / k; ++v) {
        const int32_t *r = host_table.data() + v * k;
        for (int j = 0; j < k; ++j) {
            bool dup = false;
            for (int i = 0; i < j; ++i) dup |= r[i] == r[j];
            if (r[j] < 0 || r[j] >= NE || dup) {
                delete h;
                return fail(DS4MOE_EINVAL, "create: hash_table row %lld slot %d: expert %d %s", (long long)v, j, r[j],
                            dup ? "repeated" : "out of range");
            }
        }
    }
    L.hash_table = htab;
    L.n_vocab = htab ? (int)d->n_vocab : 0;
    L.router = router, L.router_bias = bias, L.codebook = cb;
    L.router_hml = rhml, L.router_norm = rnorm;
    L.iq2_qs[0] = gq, L.iq2_qs[1] = uq, L.iq2_d[0] = gd, L.iq2_d[1] = ud;
    L.q2k_qs = dq, L.q2k_sc = dsc, L.q2k_dd = ddd;
    L.sh_gate = sg, L.sh_up = su, L.sh_down = sd;
    L.fmt = q4 ? 1 : 0;
    for (int i = 0; i < 3; ++i) L.q4_qs[i] = q4q[i], L.q4_meta[i] = q4m[i];
    if (S) {
        // the copy kernel's planes (host store -> HBM slot) and the layer as
        // the host store holds it
        ExpertPlanes &P = h->planes;
        Layer &Lh = h->Lhost;
        Lh = L;
        if (q4) {
            P.n = 6;
            for (int i = 0; i < 3; ++i) {
                const int64_t pe = i < 2 ? gu_pe : dn_pe;
                P.host[2 * i] = hq4q[i], P.hbm[2 * i] = q4q[i], P.bytes[2 * i] = pe * 128;
                P.host[2 * i + 1] = hq4m[i], P.hbm[2 * i + 1] = (uint8_t *)q4m[i], P.bytes[2 * i + 1] = pe * 16;
                Lh.q4_qs[i] = hq4q[i], Lh.q4_meta[i] = (const uint4 *)hq4m[i];
            }
        } else {
            P.n = 7;
            const uint8_t *hs[7] = {hgq, hgd, huq, hud, hdq, hdsc, hddd};
            uint8_t *ds[7] = {gq, (uint8_t *)gd, uq, (uint8_t *)ud, dq, dsc, (uint8_t *)ddd};
            const int64_t bs[7] = {gu_pe * 64, gu_pe * 2, gu_pe * 64, gu_pe * 2, dn_pe * 64, dn_pe * 16, dn_pe * 4};
            for (int i = 0; i < 7; ++i) P.host[i] = hs[i], P.hbm[i] = ds[i], P.bytes[i] = bs[i];
            Lh.iq2_qs[0] = hgq, Lh.iq2_qs[1] = huq, Lh.iq2_d[0] = (const uint16_t *)hgd, Lh.iq2_d[1] = (const uint16_t *)hud;
            Lh.q2k_qs = hdq, Lh.q2k_sc = hdsc, Lh.q2k_dd = (const uint32_t *)hddd;
        }
        h->expert_bytes = 0;
        for (int i = 0; i < P.n; ++i) h->expert_bytes += P.bytes[i];
        L.slot_of = h->cache.slot_of;
        Lh.slot_of = nullptr;
    }
    // the shared expert of large bf16 calls on hipBLASLt (without it, if the
    // library cannot be set up: the grouped kernels cover every size)
    if (d->n_shared && d->act_dtype == DS4MOE_BF16 && d->max_tokens >= SBLAS_MIN_TOK &&
        sblas_create(&h->sblas, (int)F) != 0)
        h->sblas = nullptr;
    if (h->sblas || h->W.part2) {
        // the shared expert's stream (default priority) and its fork and join
        if (hipStreamCreateWithFlags(&h->s2, hipStreamNonBlocking) != hipSuccess ||
            hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&h->ev_join, hipEventDisableTiming) != hipSuccess) {
            (void)hipGetLastError();
            delete h;
            return fail(DS4MOE_EHIP, "create: the shared expert's stream or its events");
        }
    }
    h->decode_grid = decode_grid(d->act_dtype == DS4MOE_BF16);
    // the small-batch kernels stage at most two routed slots' and two shared
    // K parts' h vectors per workgroup: a workgroup's range of down units must
    // be shorter than one slot's or one part's (n_embd / 16 units).  Its cost
    // share is at most TE (3 U + F / 256) / G shared-unit costs (routed down
    // units cost 3, shared 1; U <= SMALL_MAX_TOK k slots), so G must exceed
    // 3 U + F / 256.
    if (small_cap) {
        const int g = small_grid();
        if (g >= 3 * SMALL_MAX_TOK * (int)k + (int)(F / 256) + 1) h->small_grid = g;
    }
    if (h->decode_grid <= 0) {
        delete h;
        return fail(DS4MOE_EHIP, "create: cannot size the decode grid");
    }
    *out = h;
    g_err.clear();
    return DS4MOE_OK;
}

int ds4moe_destroy(ds4moe_t *h) {
    if (!h) return DS4MOE_OK;
    delete h;
    return DS4MOE_OK;
}

int ds4moe_set_path(ds4moe_t *h, int32_t path) {
    if (!h) return fail(DS4MOE_EINVAL, "set_path: NULL handle");
    if (path < DS4MOE_PATH_AUTO || path > DS4MOE_PATH_SMALL) return fail(DS4MOE_EINVAL, "set_path: %d", path);
    if (path == DS4MOE_PATH_GEMM && h->L.fmt == 1)
        return fail(DS4MOE_EUNSUPPORTED, "set_path: a q4 layer has no grouped GEMM path");
    if (path == DS4MOE_PATH_SMALL && !h->small_grid)
        return fail(DS4MOE_EUNSUPPORTED,
                    "set_path: the small-batch path needs bf16 activations, the 2-bit format, n_ff <= %d and "
                    "max_tokens >= 2",
                    SMALL_MAX_FF);
    h->path = path;
    return DS4MOE_OK;
}

// A bounded wait of an earlier call gave up, or a hash-routed call met a token
// id out of range (its kernel recorded the call's tag in the handle's
// host-visible status words): the handle is poisoned.
static int poll_status(ds4moe *h, const char *what) {
    if (!h->poisoned) {
        char buf[160];
        const uint32_t st = ((volatile const uint32_t *)h->status_host)[0];
        const uint32_t bad = ((volatile const uint32_t *)h->status_host)[1];
        if (st) {
            snprintf(buf, sizeof buf, "a bounded wait of an earlier call (tag %u) expired", st);
            h->poisoned = true, h->poison_why = buf;
        } else if (bad) {
            snprintf(buf, sizeof buf, "an earlier call (tag %u) had a token id outside 0..n_vocab-1", bad);
            h->poisoned = true, h->poison_why = buf;
        }
    }
    if (h->poisoned) return fail(DS4MOE_EPOISONED, "%s: handle poisoned (%s)", what, h->poison_why.c_str());
    return DS4MOE_OK;
}

// The hand-off tags come from host-side call counts, so a captured graph
// would replay one call's tags: capture is refused.
static int stream_checks(hipStream_t s, const char *what) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
        hipGetLastError();
        return fail(DS4MOE_EINVAL, "%s: invalid stream", what);
    }
    if (cs != hipStreamCaptureStatusNone)
        return fail(DS4MOE_EUNSUPPORTED, "%s: the stream is being captured into a graph (not supported)", what);
    return DS4MOE_OK;
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

static int common_checks(ds4moe *h, const void *x, int32_t n_tok, const char *what) {
    if (!h) return fail(DS4MOE_EINVAL, "%s: NULL handle", what);
    int rc = poll_status(h, what);
    if (rc) return rc;
    if (n_tok < 0 || n_tok > h->L.max_tokens)
        return fail(DS4MOE_EINVAL, "%s: n_tok %d not in 0..max_tokens (%d)", what, n_tok, h->L.max_tokens);
    if (n_tok > 0 && !x) return fail(DS4MOE_EINVAL, "%s: NULL x", what);
    if (n_tok > 0 && !aligned16(x)) return fail(DS4MOE_EINVAL, "%s: x is not 16-byte aligned", what);
    return DS4MOE_OK;
}

// A hash-routed layer needs the tokens' ids (a learned one ignores them).
static int id_checks(ds4moe *h, const int32_t *ids, int32_t n_tok, const char *what) {
    if (!h->L.hash_table || n_tok == 0) return DS4MOE_OK;
    if (!ids) return fail(DS4MOE_EINVAL, "%s: a hash-routed layer needs token ids (the *_ids entry points)", what);
    if ((uintptr_t)ids & 3u) return fail(DS4MOE_EINVAL, "%s: token_ids is not 4-byte aligned", what);
    return DS4MOE_OK;
}

static int route_impl(ds4moe_t *h, const void *x, const int32_t *ids, int32_t n_tok, int32_t *topk_idx,
                      float *topk_w, int32_t *expert_offsets, int32_t *expert_tokens, void *stream) {
    int rc = common_checks(h, x, n_tok, "route");
    if (rc) return rc;
    if ((rc = id_checks(h, ids, n_tok, "route"))) return rc;
    if (n_tok > 0 && (!topk_idx || !topk_w || !expert_offsets || !expert_tokens))
        return fail(DS4MOE_EINVAL, "route: NULL output");
    if (n_tok == 0) return DS4MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    if ((rc = stream_checks(s, "route"))) return rc;
    h->last_n_tok = n_tok;
    h->last_static = false;
    Work W = h->W;
    W.ids = ids;
    int tb = h->tbegin(TK_ROUTE, s);
    rc = check_launch(h, launch_route(h->L, W, x, n_tok, s, h->route_calls++), "route");
    h->tend(tb, s);
    if (rc) return rc;
    return check_launch(h, launch_route_export(h->L, W, n_tok, topk_idx, topk_w, expert_offsets, expert_tokens, s),
                        "route export");
}

int ds4moe_route(ds4moe_t *h, const void *x, int32_t n_tok, int32_t *topk_idx, float *topk_w,
                 int32_t *expert_offsets, int32_t *expert_tokens, void *stream) {
    return route_impl(h, x, nullptr, n_tok, topk_idx, topk_w, expert_offsets, expert_tokens, stream);
}

int ds4moe_route_ids(ds4moe_t *h, const void *x, const int32_t *token_ids, int32_t n_tok, int32_t *topk_idx,
                     float *topk_w, int32_t *expert_offsets, int32_t *expert_tokens, void *stream) {
    return route_impl(h, x, token_ids, n_tok, topk_idx, topk_w, expert_offsets, expert_tokens, stream);
}

// The expert kernels after the routing, for n <= GEMV_MAX_TOK tokens: the
// dequant-fused GEMV kernels.
static int run_gemv(ds4moe *h, const Work &W, const void *x, int n, float *out, hipStream_t s) {
    int rc = DS4MOE_OK, tb;
    if (h->L.n_shared) {
        tb = h->tbegin(TK_GU_SHARED, s);
        rc = check_launch(h, launch_gemv_gateup_shared(h->L, W, x, n, s), "gemv shared gate/up");
        h->tend(tb, s);
        if (rc) return rc;
    }
    tb = h->tbegin(TK_GU_ROUTED, s);
    rc = check_launch(h, launch_gemv_gateup_routed(h->L, W, x, n, s), "gemv routed gate/up");
    h->tend(tb, s);
    if (rc) return rc;
    tb = h->tbegin(TK_DN_ROUTED, s);
    rc = check_launch(h, launch_gemv_down_routed(h->L, W, n, out, s), "gemv routed down");
    h->tend(tb, s);
    if (rc) return rc;
    if (h->L.n_shared) {
        tb = h->tbegin(TK_DN_SHARED, s);
        rc = check_launch(h, launch_gemv_down_shared(h->L, W, n, out, s), "gemv shared down");
        h->tend(tb, s);
    }
    return rc;
}

// The expert kernels after the routing, any n: activation copies and chunk
// table, then the four grouped GEMMs.
// The shared expert of a call on the grouped path (hipBLASLt from
// SBLAS_MIN_TOK tokens, else the grouped tiles with their own partial-sum
// buffer), on the handle's second stream: forked after everything the
// caller's stream holds so far (before the routing), joined back by run_gemm
// before the routed down GEMM (both add into out; the shared one by a
// non-atomic read-modify-write).  bf16 tokens only: the tiles read x as it
// comes, where fp32 tokens need the split the activation copy makes.
static bool shared_forks(const ds4moe *h, int n) {
    if (!h->s2 || !h->L.n_shared || h->L.act_dtype != DS4MOE_BF16) return false;
    return (h->sblas && n >= SBLAS_MIN_TOK) || h->W.part2;
}
static int fork_shared(ds4moe *h, const Work &W, const void *x, int n, float *out, hipStream_t s) {
    hipStream_t s2 = h->s2;
    int rc;
    if ((rc = check_launch(h, hipEventRecord(h->ev_fork, s), "shared fork record"))) return rc;
    if ((rc = check_launch(h, hipStreamWaitEvent(s2, h->ev_fork, 0), "shared fork wait"))) return rc;
    const bool blas = h->sblas && n >= SBLAS_MIN_TOK;
    Work Ws = W;
    Ws.part = W.part2;  // the tiles' partial sums (the routed gate/up GEMM uses W.part meanwhile)
    int tb = h->tbegin(TK_GEMM_GU_SHARED, s2);
    rc = check_launch(h, blas ? sblas_gateup(h->sblas, h->L, W, x, n, s2) : launch_gemm_gateup_shared(h->L, Ws, x, n, s2),
                      "gemm shared gate/up");
    h->tend(tb, s2);
    if (rc) return rc;
    tb = h->tbegin(TK_GEMM_DN_SHARED, s2);
    rc = check_launch(h, blas ? sblas_down(h->sblas, h->L, W, n, out, s2) : launch_gemm_down_shared(h->L, Ws, n, out, s2),
                      "gemm shared down");
    h->tend(tb, s2);
    if (rc) return rc;
    return check_launch(h, hipEventRecord(h->ev_join, s2), "shared join record");
}

static int run_gemm(ds4moe *h, const Work &W, const void *x, int n, float *out, hipStream_t s, bool forked = false) {
    int tb = h->tbegin(TK_GEMM_PREP, s);
    int rc = check_launch(h, launch_gemm_prep(h->L, W, x, n, s), "gemm prep");
    h->tend(tb, s);
    if (rc) return rc;
    tb = h->tbegin(TK_GEMM_GU_ROUTED, s);
    rc = check_launch(h, launch_gemm_gateup_routed(h->L, W, n, s), "gemm routed gate/up");
    h->tend(tb, s);
    if (rc) return rc;
    const bool blas = h->sblas && n >= SBLAS_MIN_TOK;
    if (h->L.n_shared && !forked) {
        tb = h->tbegin(TK_GEMM_GU_SHARED, s);
        rc = check_launch(h, blas ? sblas_gateup(h->sblas, h->L, W, x, n, s) : launch_gemm_gateup_shared(h->L, W, x, n, s),
                          "gemm shared gate/up");
        h->tend(tb, s);
        if (rc) return rc;
    }
    // the forked shared expert has added into out before the routed atomics start
    if (forked && (rc = check_launch(h, hipStreamWaitEvent(s, h->ev_join, 0), "shared join wait"))) return rc;
    tb = h->tbegin(TK_GEMM_DN_ROUTED, s);
    rc = check_launch(h, launch_gemm_down_routed(h->L, W, n, out, s), "gemm routed down");
    h->tend(tb, s);
    if (rc) return rc;
    if (h->L.n_shared && !forked) {
        tb = h->tbegin(TK_GEMM_DN_SHARED, s);
        rc = check_launch(h, blas ? sblas_down(h->sblas, h->L, W, n, out, s) : launch_gemm_down_shared(h->L, W, n, out, s),
                          "gemm shared down");
        h->tend(tb, s);
    }
    return rc;
}

// The expert kernels after the routing for 2..SMALL_MAX_TOK bf16 tokens: the
// two persistent small-batch kernels (gate/up sums into one buffer, then the
// down projections, which also clear the other buffer for the next call).
static bool small_ok(const ds4moe *h, int n) { return h->small_grid > 0 && n >= 2 && n <= SMALL_MAX_TOK; }

static int run_small(ds4moe *h, const Work &W, const void *x, int n, float *out, hipStream_t s) {
    const size_t zn = small_sum_floats(h->L);
    float *gu = W.sgu + (size_t)h->small_parity * zn, *gz = W.sgu + (size_t)(1 - h->small_parity) * zn;
    int tb = h->tbegin(TK_SMALL_GU, s);
    int rc = check_launch(h, launch_small_gateup(h->L, W, x, n, gu, h->small_grid, s), "small-batch gate/up");
    h->tend(tb, s);
    if (rc) return rc;
    tb = h->tbegin(TK_SMALL_DN, s);
    rc = check_launch(h, launch_small_down(h->L, W, gu, gz, n, out, h->small_grid, s), "small-batch down");
    h->tend(tb, s);
    if (rc) return rc;
    h->small_parity ^= 1;
    return DS4MOE_OK;
}

static int run_route(ds4moe *h, const Work &W, const void *x, int n, hipStream_t s, bool lists = true) {
    int tb = h->tbegin(TK_ROUTE, s);
    int rc = check_launch(h, launch_route(h->L, W, x, n, s, h->route_calls++, lists), "route");
    h->tend(tb, s);
    return rc;
}

// Host-resident experts: after the routing, the cache update and the copy of
// the missed experts into their HBM slots.
static int run_cache(ds4moe *h, const Work &W, hipStream_t s) {
    int tb = h->tbegin(TK_CACHE, s);
    int rc = check_launch(h, launch_cache_update(h->L, W, h->cache, h->expert_bytes, s), "cache update");
    if (!rc) rc = check_launch(h, launch_cache_fill(h->planes, h->cache, s), "cache fill");
    h->tend(tb, s);
    return rc;
}

// A layer with host-resident experts: the call in sub-calls whose distinct
// experts fit in the cache's slots (at most slots / top_k tokens each, unless
// the slots hold every expert), each routed, cached and computed in turn.
static int forward_cached(ds4moe *h, const void *x, const int32_t *ids, int n_tok, float *out, hipStream_t s) {
    const Layer &L = h->L;
    int chunk = h->cache.slots >= L.n_expert ? n_tok : std::max(1, h->cache.slots / L.top_k);
    if (L.fmt == 1 || h->path == DS4MOE_PATH_GEMV) chunk = std::min(chunk, GEMV_MAX_TOK);
    if (h->path == DS4MOE_PATH_SMALL) chunk = std::min(chunk, SMALL_MAX_TOK);
    h->last_n_tok = chunk >= n_tok ? n_tok : -1;
    h->last_static = false;
    const size_t xb = L.act_dtype == DS4MOE_BF16 ? 2 : 4;
    for (int c0 = 0; c0 < n_tok; c0 += chunk) {
        const int n = std::min(chunk, n_tok - c0);
        const void *xc = (const char *)x + (size_t)c0 * L.n_embd * xb;
        float *oc = out + (size_t)c0 * L.n_embd;
        Work W = h->W;
        W.ids = ids ? ids + c0 : nullptr;
        int rc = run_route(h, W, xc, n, s);
        if (!rc) rc = run_cache(h, W, s);
        if (rc) return rc;
        if (n == 1 && L.fmt == 0 && (h->path == DS4MOE_PATH_AUTO || h->path == DS4MOE_PATH_SMALL)) {
            // one token: the fused decode kernel, taking the routing from the
            // router kernel (its own router phase would come after the cache step)
            int tf = h->tbegin(TK_FUSED, s);
            rc = check_launch(h, launch_decode_fused(L, W, xc, oc, h->decode_grid, h->decode_calls, s, true),
                              "fused decode");
            h->decode_calls += 1;
            h->tend(tf, s);
            if (rc) return rc;
            continue;
        }
        bool gemv = n <= GEMV_MAX_TOK && (L.fmt == 1 || h->path == DS4MOE_PATH_GEMV ||
                                          (h->path == DS4MOE_PATH_AUTO && L.act_dtype == DS4MOE_F32));
        const bool small = !gemv && small_ok(h, n) && (h->path == DS4MOE_PATH_AUTO || h->path == DS4MOE_PATH_SMALL);
        rc = L.fmt == 1 ? run_q4_experts(h, W, xc, n, oc, s, true)
             : gemv     ? run_gemv(h, W, xc, n, oc, s)
             : small    ? run_small(h, W, xc, n, oc, s)
                        : run_gemm(h, W, xc, n, oc, s);
        if (rc) return rc;
    }
    return DS4MOE_OK;
}

static int forward_impl(ds4moe_t *h, const void *x, const int32_t *ids, int32_t n_tok, float *out, void *stream) {
    int rc = common_checks(h, x, n_tok, "forward");
    if (rc) return rc;
    if ((rc = id_checks(h, ids, n_tok, "forward"))) return rc;
    if (n_tok > 0 && !out) return fail(DS4MOE_EINVAL, "forward: NULL out");
    if (n_tok > 0 && !aligned16(out)) return fail(DS4MOE_EINVAL, "forward: out is not 16-byte aligned");
    if (n_tok == 0) return DS4MOE_OK;
    if ((rc = stream_checks((hipStream_t)stream, "forward"))) return rc;
    hipStream_t s = (hipStream_t)stream;
    if (h->cache.slots) return forward_cached(h, x, ids, n_tok, out, s);
    if (h->L.fmt == 1) {
        // q4: the GEMV kernels (set_path refuses the GEMM path), in chunks of
        // up to GEMV_MAX_TOK tokens; the routing of a call of more tokens is
        // not kept for ds4moe_last_routing
        h->last_n_tok = n_tok <= GEMV_MAX_TOK ? n_tok : -1;
        h->last_static = false;
        const size_t xb = h->L.act_dtype == DS4MOE_BF16 ? 2 : 4;
        for (int c0 = 0; c0 < n_tok; c0 += GEMV_MAX_TOK) {
            const int nc = std::min(GEMV_MAX_TOK, n_tok - c0);
            const void *xc = (const char *)x + (size_t)c0 * h->L.n_embd * xb;
            float *oc = out + (size_t)c0 * h->L.n_embd;
            Work Wc = h->W;
            Wc.ids = ids ? ids + c0 : nullptr;
            if ((rc = run_q4_chunk(h, Wc, xc, nc, oc, h->route_calls++, s, true))) return rc;
        }
        return DS4MOE_OK;
    }
    int path = h->path;
    // one token: the fused decode kernel; 2..SMALL_MAX_TOK bf16 tokens: the
    // small-batch kernels; more: the grouped GEMMs.  fp32 activations of up to
    // 4 tokens keep the GEMV kernels, which do not round them to fp16.
    if (path == DS4MOE_PATH_AUTO)
        path = n_tok == 1 || (n_tok <= GEMV_MAX_TOK && h->L.act_dtype == DS4MOE_F32) ? DS4MOE_PATH_GEMV
               : small_ok(h, n_tok)                                                  ? DS4MOE_PATH_SMALL
                                                                                     : DS4MOE_PATH_GEMM;
    if (path == DS4MOE_PATH_GEMV && n_tok > GEMV_MAX_TOK)
        return fail(DS4MOE_EUNSUPPORTED, "forward: GEMV path takes at most %d tokens (got %d)", GEMV_MAX_TOK, n_tok);
    if (path == DS4MOE_PATH_SMALL && (n_tok < 2 || !small_ok(h, n_tok)))
        return fail(DS4MOE_EUNSUPPORTED, "forward: the small-batch path takes 2..%d tokens (got %d)", SMALL_MAX_TOK,
                    n_tok);
    if (path == DS4MOE_PATH_GEMM && !gemm_available())
        return fail(DS4MOE_EUNSUPPORTED, "forward: the grouped GEMM path is not available in this build");
    h->last_n_tok = n_tok;
    h->last_static = false;
    Work W = h->W;
    W.ids = ids;
    if (path == DS4MOE_PATH_GEMV && n_tok == 1) {
        // the whole block for one token in one persistent launch
        int tf = h->tbegin(TK_FUSED, s);
        rc = check_launch(h, launch_decode_fused(h->L, W, x, out, h->decode_grid, h->decode_calls, s),
                          "fused decode");
        h->decode_calls += 1;
        h->tend(tf, s);
        return rc;
    }
    // the small-batch kernels build the per-expert lists themselves
    // a large call's shared expert runs beside the routing and routed gate/up
    const bool forked = path == DS4MOE_PATH_GEMM && shared_forks(h, n_tok);
    if (forked && (rc = fork_shared(h, W, x, n_tok, out, s))) return rc;
    if ((rc = run_route(h, W, x, n_tok, s, path != DS4MOE_PATH_SMALL))) return rc;
    return path == DS4MOE_PATH_GEMV    ? run_gemv(h, W, x, n_tok, out, s)
           : path == DS4MOE_PATH_SMALL ? run_small(h, W, x, n_tok, out, s)
                                       : run_gemm(h, W, x, n_tok, out, s, forked);
}

int ds4moe_forward(ds4moe_t *h, const void *x, int32_t n_tok, float *out, void *stream) {
    return forward_impl(h, x, nullptr, n_tok, out, stream);
}

int ds4moe_forward_ids(ds4moe_t *h, const void *x, const int32_t *token_ids, int32_t n_tok, float *out,
                       void *stream) {
    return forward_impl(h, x, token_ids, n_tok, out, stream);
}

int ds4moe_forward_static(ds4moe_t *h, const void *x, int32_t n_tok, float *out, void *stream) {
    int rc = common_checks(h, x, n_tok, "forward_static");
    if (rc) return rc;
    if (h->L.hash_table)
        return fail(DS4MOE_EUNSUPPORTED, "forward_static: a hash-routed layer takes token ids (ds4moe_forward_ids)");
    if (h->cache.slots)
        return fail(DS4MOE_EUNSUPPORTED, "forward_static: a layer with host-resident experts needs ds4moe_forward");
    if (n_tok > STATIC_MAX_TOK)
        return fail(DS4MOE_EINVAL, "forward_static: n_tok %d beyond the static scratch's %d tokens", n_tok,
                    STATIC_MAX_TOK);
    if (n_tok > 0 && !out) return fail(DS4MOE_EINVAL, "forward_static: NULL out");
    if (n_tok > 0 && !aligned16(out)) return fail(DS4MOE_EINVAL, "forward_static: out is not 16-byte aligned");
    if (n_tok == 0) return DS4MOE_OK;
    if (h->static_need > STATIC_BYTES)
        return fail(DS4MOE_EINVAL, "forward_static: this layer needs %zu bytes of scratch, the static array holds %zu",
                    h->static_need, STATIC_BYTES);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != h->device) {
        hipGetLastError();
        return fail(DS4MOE_EINVAL, "forward_static: the handle's device %d is not the current device %d", h->device,
                    dev);
    }
    hipStream_t s = (hipStream_t)stream;
    if ((rc = stream_checks(s, "forward_static"))) return rc;
    Work S = h->Wst;
    S.spin_limit = h->W.spin_limit;
    S.want_xor = h->W.want_xor;
    const unsigned long long ep = g_static_calls[dev].fetch_add(1);
    h->last_n_tok = n_tok;
    h->last_static = true;
    if (h->L.fmt == 1) {
        // the router's tickets start at zero
        rc = check_launch(h, launch_fill_u32((uint32_t *)S.counters, 64, 0u, s), "forward_static clear");
        if (rc) return rc;
        return run_q4_chunk(h, S, x, n_tok, out, ep, s, false);
    }
    if (n_tok == 1)
        return check_launch(h, launch_decode_fused(h->L, S, x, out, h->decode_grid, ep, s), "forward_static decode");
    // the router's tickets start at zero
    rc = check_launch(h, launch_fill_u32((uint32_t *)S.counters, 64, 0u, s), "forward_static clear");
    if (rc) return rc;
    rc = check_launch(h, launch_route(h->L, S, x, n_tok, s, ep), "forward_static route");
    if (rc) return rc;
    if (h->L.n_shared) {
        rc = check_launch(h, launch_gemv_gateup_shared(h->L, S, x, n_tok, s), "forward_static shared gate/up");
        if (rc) return rc;
    }
    rc = check_launch(h, launch_gemv_gateup_routed(h->L, S, x, n_tok, s), "forward_static routed gate/up");
    if (rc) return rc;
    rc = check_launch(h, launch_gemv_down_routed(h->L, S, n_tok, out, s), "forward_static routed down");
    if (rc) return rc;
    if (h->L.n_shared) rc = check_launch(h, launch_gemv_down_shared(h->L, S, n_tok, out, s), "forward_static shared down");
    return rc;
}

int ds4moe_dequantize(ds4moe_t *h, int32_t expert, int32_t which, float *dst, void *stream) {
    if (!h) return fail(DS4MOE_EINVAL, "dequantize: NULL handle");
    if (h->poisoned) return fail(DS4MOE_EPOISONED, "dequantize: handle poisoned");
    if (expert < 0 || expert >= h->L.n_expert) return fail(DS4MOE_EINVAL, "dequantize: expert %d", expert);
    if (which < 0 || which > 2) return fail(DS4MOE_EINVAL, "dequantize: which %d", which);
    if (!dst) return fail(DS4MOE_EINVAL, "dequantize: NULL dst");
    hipStream_t s = (hipStream_t)stream;
    // with host-resident experts, decoded from the host store (every expert)
    const Layer &L = h->cache.slots ? h->Lhost : h->L;
    hipError_t e = L.fmt == 1 ? launch_dequant_q4k(L, which, expert, dst, s)
                   : (which < 2) ? launch_dequant_iq2(L, which, expert, dst, s)
                                 : launch_dequant_q2k(L, expert, dst, s);
    return check_launch(h, e, "dequantize");
}

int ds4moe_debug_gemm_b(ds4moe_t *h, int32_t expert, int32_t which, float *dst, void *stream) {
    if (!h) return fail(DS4MOE_EINVAL, "debug_gemm_b: NULL handle");
    if (h->poisoned) return fail(DS4MOE_EPOISONED, "debug_gemm_b: handle poisoned");
    if (h->L.fmt == 1) return fail(DS4MOE_EUNSUPPORTED, "debug_gemm_b: a q4 layer has no grouped GEMM path");
    if (expert < 0 || expert >= h->L.n_expert) return fail(DS4MOE_EINVAL, "debug_gemm_b: expert %d", expert);
    if (which < 0 || which > 2) return fail(DS4MOE_EINVAL, "debug_gemm_b: which %d", which);
    if (!dst) return fail(DS4MOE_EINVAL, "debug_gemm_b: NULL dst");
    const Layer &L = h->cache.slots ? h->Lhost : h->L;
    return check_launch(h, launch_debug_gemm_b(L, which, expert, dst, (hipStream_t)stream), "debug_gemm_b");
}

int ds4moe_rmsnorm(const float *hin, int32_t n_tok, int32_t n_embd, double eps, uint16_t *x_bf16, void *stream) {
    if (n_tok < 0 || n_embd < 1 || n_embd > 65536 || !(eps >= 0.0))
        return fail(DS4MOE_EINVAL, "rmsnorm: n_tok %d, n_embd %d, eps %g", n_tok, n_embd, eps);
    if (n_tok == 0) return DS4MOE_OK;
    if (!hin || !x_bf16) return fail(DS4MOE_EINVAL, "rmsnorm: NULL pointer");
    hipError_t e = launch_rmsnorm(hin, n_tok, n_embd, eps, x_bf16, (hipStream_t)stream);
    if (e != hipSuccess) return fail(DS4MOE_EHIP, "rmsnorm: %s", hipGetErrorString(e));
    return DS4MOE_OK;
}

static int forward_stack_impl(ds4moe_t *const *layers, int32_t n_layers, float *h, const int32_t *ids,
                              int32_t n_tok, double eps, uint16_t *x_bf16, void *stream) {
    if (!layers || n_layers < 1) return fail(DS4MOE_EINVAL, "forward_stack: no layers");
    if (n_tok < 0 || !(eps >= 0.0)) return fail(DS4MOE_EINVAL, "forward_stack: n_tok %d, eps %g", n_tok, eps);
    if (n_tok > 0 && (!h || !x_bf16)) return fail(DS4MOE_EINVAL, "forward_stack: NULL h or x");
    if (n_tok > 0 && (!aligned16(h) || !aligned16(x_bf16)))
        return fail(DS4MOE_EINVAL, "forward_stack: h or x is not 16-byte aligned");
    // every layer is checked before anything is enqueued
    for (int l = 0; l < n_layers; ++l) {
        ds4moe *d = layers[l];
        int rc = common_checks(d, x_bf16, n_tok, "forward_stack");
        if (rc) return fail(rc, "forward_stack: layer %d: %s", l, g_err.c_str());
        if (d->L.act_dtype != DS4MOE_BF16)
            return fail(DS4MOE_EINVAL, "forward_stack: layer %d takes fp32 activations (needs bf16)", l);
        if (d->L.n_embd != layers[0]->L.n_embd)
            return fail(DS4MOE_EINVAL, "forward_stack: layer %d has n_embd %d, layer 0 %d", l, d->L.n_embd,
                        layers[0]->L.n_embd);
        if ((rc = id_checks(d, ids, n_tok, "forward_stack"))) return fail(rc, "forward_stack: layer %d: %s", l, g_err.c_str());
    }
    if (n_tok == 0) return DS4MOE_OK;
    {
        int rc = stream_checks((hipStream_t)stream, "forward_stack");
        if (rc) return rc;
    }
    const int E = layers[0]->L.n_embd;
    for (int l = 0; l < n_layers; ++l) {
        hipError_t e = launch_rmsnorm(h, n_tok, E, eps, x_bf16, (hipStream_t)stream);
        if (e != hipSuccess) return fail(DS4MOE_EHIP, "forward_stack: layer %d rmsnorm: %s", l, hipGetErrorString(e));
        int rc = forward_impl(layers[l], x_bf16, ids, n_tok, h, stream);
        if (rc) return fail(rc, "forward_stack: layer %d: %s", l, g_err.c_str());
    }
    return DS4MOE_OK;
}

int ds4moe_forward_stack(ds4moe_t *const *layers, int32_t n_layers, float *h, int32_t n_tok, double eps,
                         uint16_t *x_bf16, void *stream) {
    return forward_stack_impl(layers, n_layers, h, nullptr, n_tok, eps, x_bf16, stream);
}

int ds4moe_forward_stack_ids(ds4moe_t *const *layers, int32_t n_layers, float *h, const int32_t *token_ids,
                             int32_t n_tok, double eps, uint16_t *x_bf16, void *stream) {
    return forward_stack_impl(layers, n_layers, h, token_ids, n_tok, eps, x_bf16, stream);
}

int ds4moe_last_routing(ds4moe_t *h, int32_t n_tok, int32_t *topk_idx, float *topk_w, int32_t *expert_offsets,
                        int32_t *expert_tokens, void *stream) {
    if (!h) return fail(DS4MOE_EINVAL, "last_routing: NULL handle");
    int rc = poll_status(h, "last_routing");
    if (rc) return rc;
    if (h->last_n_tok < 1 || n_tok != h->last_n_tok)
        return fail(DS4MOE_EINVAL, "last_routing: n_tok %d, the latest forward/route call had %d", n_tok,
                    h->last_n_tok);
    if (!topk_idx || !topk_w || !expert_offsets || !expert_tokens)
        return fail(DS4MOE_EINVAL, "last_routing: NULL output");
    hipStream_t s = (hipStream_t)stream;
    if ((rc = stream_checks(s, "last_routing"))) return rc;
    return check_launch(h, launch_route_export(h->L, h->last_static ? h->Wst : h->W, n_tok, topk_idx, topk_w,
                                               expert_offsets, expert_tokens, s),
                        "last_routing export");
}

int ds4moe_status(ds4moe_t *h) {
    if (!h) return fail(DS4MOE_EINVAL, "status: NULL handle");
    return poll_status(h, "status");
}

int ds4moe_set_wait_limit(ds4moe_t *h, int32_t max_polls, int32_t force_expire) {
    if (!h) return fail(DS4MOE_EINVAL, "set_wait_limit: NULL handle");
    if (max_polls < 0) return fail(DS4MOE_EINVAL, "set_wait_limit: max_polls %d", max_polls);
    h->W.spin_limit = max_polls ? max_polls : DEFAULT_SPIN_LIMIT;
    h->W.want_xor = force_expire ? 0x80000000u : 0u;
    return DS4MOE_OK;
}

int ds4moe_cache_stats(ds4moe_t *h, int64_t *stats, void *stream) {
    if (!h || !stats) return fail(DS4MOE_EINVAL, "cache_stats: NULL argument");
    if (!h->cache.slots) return fail(DS4MOE_EUNSUPPORTED, "cache_stats: the layer's experts are all resident in HBM");
    hipStream_t s = (hipStream_t)stream;
    unsigned long long v[4];
    if (hipMemcpyAsync(v, h->cache.stats, sizeof v, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess) {
        hipGetLastError();
        return fail(DS4MOE_EHIP, "cache_stats: copy");
    }
    for (int i = 0; i < 4; ++i) stats[i] = (int64_t)v[i];
    return DS4MOE_OK;
}

int ds4moe_cache_slots(ds4moe_t *h, int32_t *slot_expert, void *stream) {
    if (!h || !slot_expert) return fail(DS4MOE_EINVAL, "cache_slots: NULL argument");
    if (!h->cache.slots) return fail(DS4MOE_EUNSUPPORTED, "cache_slots: the layer's experts are all resident in HBM");
    hipStream_t s = (hipStream_t)stream;
    if (hipMemcpyAsync(slot_expert, h->cache.slot_expert, (size_t)h->cache.slots * 4, hipMemcpyDeviceToHost, s) !=
            hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess) {
        hipGetLastError();
        return fail(DS4MOE_EHIP, "cache_slots: copy");
    }
    return DS4MOE_OK;
}

int ds4moe_timing_enable(ds4moe_t *h, int32_t enable) {
    if (!h) return fail(DS4MOE_EINVAL, "timing_enable: NULL handle");
    if (enable && h->events.empty()) {
        h->events.resize(TIMING_EVENTS);
        h->event_kind.resize(TIMING_EVENTS / 2);
        for (auto &e : h->events)
            if (hipEventCreate(&e) != hipSuccess) return fail(DS4MOE_EHIP, "timing_enable: hipEventCreate");
    }
    h->timing = enable != 0;
    h->n_events = 0;
    for (int i = 0; i < TIMING_SLOTS; ++i) h->ms[i] = 0.0, h->counts[i] = 0;
    return DS4MOE_OK;
}

int ds4moe_timing_read(ds4moe_t *h, double *ms, int64_t *counts) {
    if (!h || !ms || !counts) return fail(DS4MOE_EINVAL, "timing_read: NULL argument");
    for (int i = 0; i + 1 < h->n_events; i += 2) {
        if (hipEventSynchronize(h->events[i + 1]) != hipSuccess) return fail(DS4MOE_EHIP, "timing_read: sync");
        float t = 0.0f;
        hipEventElapsedTime(&t, h->events[i], h->events[i + 1]);
        int kind = h->event_kind[i / 2];
        h->ms[kind] += t;
        h->counts[kind] += 1;
    }
    h->n_events = 0;
    for (int i = 0; i < TIMING_SLOTS; ++i) ms[i] = h->ms[i], counts[i] = h->counts[i];
    return DS4MOE_OK;
}

}  // extern "C"

// GEMM path entry points are provided by gemm.hip.
