// ds4moe.hip - host side of libds4moe.so: the C ABI declared in include/ds4moe.h.
//
// create() owns every device buffer of a layer (repacked experts, router and
// shared-expert copies, workspace); route()/forward() only validate and enqueue
// kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
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
constexpr int TIMING_EVENTS = 4096;

}  // namespace

struct ds4moe {
    Layer L{};
    Work W{};
    int path = DS4MOE_PATH_AUTO;
    int decode_grid = 0;    // workgroups of the persistent decode kernel
    unsigned long long decode_calls = 0;  // fused launches so far (the phase counters' epoch)
    unsigned long long route_calls = 0;   // routing launches so far (the router hand-off tag)
    bool poisoned = false;
    int device = 0;
    std::vector<void *> allocs;
    // timing
    bool timing = false;
    std::vector<hipEvent_t> events;  // pairs
    std::vector<int> event_kind;
    int n_events = 0;
    double ms[TIMING_SLOTS] = {};
    int64_t counts[TIMING_SLOTS] = {};

    ~ds4moe() {
        for (void *p : allocs) hipFree(p);
        for (hipEvent_t e : events) hipEventDestroy(e);
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
        return fail(DS4MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
    }
    return DS4MOE_OK;
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
    if (!d->router || !d->gate || !d->up || !d->down || !d->codebook)
        return fail(DS4MOE_EINVAL, "create: NULL router/gate/up/down/codebook");
    if (d->n_shared && (!d->sh_gate || !d->sh_up || !d->sh_down))
        return fail(DS4MOE_EINVAL, "create: n_shared = 1 but a shared-expert pointer is NULL");

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
    uint8_t *gq = (uint8_t *)A(gu_blocks * 64), *uq = (uint8_t *)A(gu_blocks * 64);
    uint16_t *gd = (uint16_t *)A(gu_blocks * 2), *ud = (uint16_t *)A(gu_blocks * 2);
    uint8_t *dq = (uint8_t *)A(dn_blocks * 64), *dsc = (uint8_t *)A(dn_blocks * 16);
    uint32_t *ddd = (uint32_t *)A(dn_blocks * 4);
    uint16_t *sg = nullptr, *su = nullptr, *sd = nullptr;
    if (d->n_shared) {
        sg = (uint16_t *)A(F * E * 2);
        su = (uint16_t *)A(F * E * 2);
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
    size_t o_chunks = carve((size_t)gemm_max_chunks((int)T, (int)NE, (int)k) * 16), o_nch = carve(4);
    size_t o_ecnt = carve(MAX_EXPERT * 4), o_rest = carve(4 * T * NE * 4), o_rtag = carve(4 * MAX_EXPERT * 8);
    size_t o_htag = carve((size_t)(k + 1) * F * 8);
    size_t o_ltag = carve(64 * MAX_EXPERT * 8), o_itag = carve(64 * MAX_TOPK * 8);
    char *ws = (char *)A(off);
    if (err != hipSuccess) {
        delete h;
        hipGetLastError();
        return fail(DS4MOE_ENOMEM, "create: device allocation failed (%s)", hipGetErrorString(err));
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
    W.chunks = (int4 *)(ws + o_chunks);
    W.nchunks = (int32_t *)(ws + o_nch);
    W.ecount = (int32_t *)(ws + o_ecnt);
    W.rest = (float *)(ws + o_rest);
    W.rtag = (unsigned long long *)(ws + o_rtag);
    W.htag = (unsigned long long *)(ws + o_htag);
    W.ltag = (unsigned long long *)(ws + o_ltag);
    W.itag = (unsigned long long *)(ws + o_itag);

#define CK(call)                                                                                      \
    do {                                                                                              \
        hipError_t e_ = (call);                                                                       \
        if (e_ != hipSuccess) {                                                                       \
            delete h;                                                                                 \
            return fail(DS4MOE_EHIP, "create: %s: %s", #call, hipGetErrorString(e_));                 \
        }                                                                                             \
    } while (0)
    CK(hipMemsetAsync(ws, 0, off, s));
    CK(hipMemcpyAsync(router, d->router, NE * E * 4, hipMemcpyDeviceToDevice, s));
    if (bias) CK(hipMemcpyAsync(bias, d->router_bias, NE * 4, hipMemcpyDeviceToDevice, s));
    CK(launch_router_prep(router, (int)NE, (int)E, rhml, rnorm, s));
    CK(hipMemcpyAsync(cb, d->codebook, 512, hipMemcpyHostToDevice, s));
    if (d->n_shared) {
        CK(hipMemcpyAsync(sg, d->sh_gate, F * E * 2, hipMemcpyDeviceToDevice, s));
        CK(hipMemcpyAsync(su, d->sh_up, F * E * 2, hipMemcpyDeviceToDevice, s));
        CK(hipMemcpyAsync(sd, d->sh_down, E * F * 2, hipMemcpyDeviceToDevice, s));
    }
    CK(launch_repack_iq2((const uint8_t *)d->gate, gu_blocks, gq, gd, s));
    CK(launch_repack_iq2((const uint8_t *)d->up, gu_blocks, uq, ud, s));
    CK(launch_repack_q2k((const uint8_t *)d->down, dn_blocks, dq, dsc, ddd, s));
    CK(hipStreamSynchronize(s));
#undef CK
    L.router = router, L.router_bias = bias, L.codebook = cb;
    L.router_hml = rhml, L.router_norm = rnorm;
    L.iq2_qs[0] = gq, L.iq2_qs[1] = uq, L.iq2_d[0] = gd, L.iq2_d[1] = ud;
    L.q2k_qs = dq, L.q2k_sc = dsc, L.q2k_dd = ddd;
    L.sh_gate = sg, L.sh_up = su, L.sh_down = sd;
    h->decode_grid = decode_grid(d->act_dtype == DS4MOE_BF16);
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
    if (path < DS4MOE_PATH_AUTO || path > DS4MOE_PATH_GEMM) return fail(DS4MOE_EINVAL, "set_path: %d", path);
    h->path = path;
    return DS4MOE_OK;
}

static int common_checks(ds4moe *h, const void *x, int32_t n_tok, const char *what) {
    if (!h) return fail(DS4MOE_EINVAL, "%s: NULL handle", what);
    if (h->poisoned) return fail(DS4MOE_EPOISONED, "%s: handle poisoned by an earlier HIP error", what);
    if (n_tok < 0 || n_tok > h->L.max_tokens)
        return fail(DS4MOE_EINVAL, "%s: n_tok %d not in 0..max_tokens (%d)", what, n_tok, h->L.max_tokens);
    if (n_tok > 0 && !x) return fail(DS4MOE_EINVAL, "%s: NULL x", what);
    return DS4MOE_OK;
}

int ds4moe_route(ds4moe_t *h, const void *x, int32_t n_tok, int32_t *topk_idx, float *topk_w,
                 int32_t *expert_offsets, int32_t *expert_tokens, void *stream) {
    int rc = common_checks(h, x, n_tok, "route");
    if (rc) return rc;
    if (n_tok > 0 && (!topk_idx || !topk_w || !expert_offsets || !expert_tokens))
        return fail(DS4MOE_EINVAL, "route: NULL output");
    if (n_tok == 0) return DS4MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    int tb = h->tbegin(TK_ROUTE, s);
    rc = check_launch(h, launch_route(h->L, h->W, x, n_tok, s, h->route_calls++), "route");
    h->tend(tb, s);
    if (rc) return rc;
    return check_launch(h, launch_route_export(h->L, h->W, n_tok, topk_idx, topk_w, expert_offsets, expert_tokens, s),
                        "route export");
}

int ds4moe_forward(ds4moe_t *h, const void *x, int32_t n_tok, float *out, void *stream) {
    int rc = common_checks(h, x, n_tok, "forward");
    if (rc) return rc;
    if (n_tok > 0 && !out) return fail(DS4MOE_EINVAL, "forward: NULL out");
    if (n_tok == 0) return DS4MOE_OK;
    int path = h->path;
    // one token: the fused decode kernel; more: the grouped GEMMs, which at 2-4
    // tokens (K split over more workgroups) also beat the GEMV kernels.  fp32
    // activations of up to 4 tokens keep the GEMV kernels, which do not round
    // them to fp16.
    if (path == DS4MOE_PATH_AUTO)
        path = (n_tok == 1 || (n_tok <= GEMV_MAX_TOK && h->L.act_dtype == DS4MOE_F32)) ? DS4MOE_PATH_GEMV
                                                                                      : DS4MOE_PATH_GEMM;
    if (path == DS4MOE_PATH_GEMV && n_tok > GEMV_MAX_TOK)
        return fail(DS4MOE_EUNSUPPORTED, "forward: GEMV path takes at most %d tokens (got %d)", GEMV_MAX_TOK, n_tok);
    if (path == DS4MOE_PATH_GEMM && !gemm_available())
        return fail(DS4MOE_EUNSUPPORTED, "forward: the grouped GEMM path is not available in this build");
    hipStream_t s = (hipStream_t)stream;
    if (path == DS4MOE_PATH_GEMV && n_tok == 1) {
        // the whole block for one token in one persistent launch
        int tf = h->tbegin(TK_FUSED, s);
        rc = check_launch(h, launch_decode_fused(h->L, h->W, x, out, h->decode_grid, h->decode_calls, s),
                          "fused decode");
        h->decode_calls += 1;
        h->tend(tf, s);
        return rc;
    }
    int tb = h->tbegin(TK_ROUTE, s);
    rc = check_launch(h, launch_route(h->L, h->W, x, n_tok, s, h->route_calls++), "route");
    h->tend(tb, s);
    if (rc) return rc;
    if (path == DS4MOE_PATH_GEMV) {
        if (h->L.n_shared) {
            tb = h->tbegin(TK_GU_SHARED, s);
            rc = check_launch(h, launch_gemv_gateup_shared(h->L, h->W, x, n_tok, s), "gemv shared gate/up");
            h->tend(tb, s);
            if (rc) return rc;
        }
        tb = h->tbegin(TK_GU_ROUTED, s);
        rc = check_launch(h, launch_gemv_gateup_routed(h->L, h->W, x, n_tok, s), "gemv routed gate/up");
        h->tend(tb, s);
        if (rc) return rc;
        tb = h->tbegin(TK_DN_ROUTED, s);
        rc = check_launch(h, launch_gemv_down_routed(h->L, h->W, n_tok, out, s), "gemv routed down");
        h->tend(tb, s);
        if (rc) return rc;
        if (h->L.n_shared) {
            tb = h->tbegin(TK_DN_SHARED, s);
            rc = check_launch(h, launch_gemv_down_shared(h->L, h->W, n_tok, out, s), "gemv shared down");
            h->tend(tb, s);
        }
        return rc;
    }
    // batched path: activation copies and chunk table, then the four grouped GEMMs
    tb = h->tbegin(TK_GEMM_PREP, s);
    rc = check_launch(h, launch_gemm_prep(h->L, h->W, x, n_tok, s), "gemm prep");
    h->tend(tb, s);
    if (rc) return rc;
    tb = h->tbegin(TK_GEMM_GU_ROUTED, s);
    rc = check_launch(h, launch_gemm_gateup_routed(h->L, h->W, n_tok, s), "gemm routed gate/up");
    h->tend(tb, s);
    if (rc) return rc;
    if (h->L.n_shared) {
        tb = h->tbegin(TK_GEMM_GU_SHARED, s);
        rc = check_launch(h, launch_gemm_gateup_shared(h->L, h->W, x, n_tok, s), "gemm shared gate/up");
        h->tend(tb, s);
        if (rc) return rc;
    }
    tb = h->tbegin(TK_GEMM_DN_ROUTED, s);
    rc = check_launch(h, launch_gemm_down_routed(h->L, h->W, n_tok, out, s), "gemm routed down");
    h->tend(tb, s);
    if (rc) return rc;
    if (h->L.n_shared) {
        tb = h->tbegin(TK_GEMM_DN_SHARED, s);
        rc = check_launch(h, launch_gemm_down_shared(h->L, h->W, n_tok, out, s), "gemm shared down");
        h->tend(tb, s);
    }
    return rc;
}

int ds4moe_dequantize(ds4moe_t *h, int32_t expert, int32_t which, float *dst, void *stream) {
    if (!h) return fail(DS4MOE_EINVAL, "dequantize: NULL handle");
    if (h->poisoned) return fail(DS4MOE_EPOISONED, "dequantize: handle poisoned");
    if (expert < 0 || expert >= h->L.n_expert) return fail(DS4MOE_EINVAL, "dequantize: expert %d", expert);
    if (which < 0 || which > 2) return fail(DS4MOE_EINVAL, "dequantize: which %d", which);
    if (!dst) return fail(DS4MOE_EINVAL, "dequantize: NULL dst");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = (which < 2) ? launch_dequant_iq2(h->L, which, expert, dst, s) : launch_dequant_q2k(h->L, expert, dst, s);
    return check_launch(h, e, "dequantize");
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

int ds4moe_forward_stack(ds4moe_t *const *layers, int32_t n_layers, float *h, int32_t n_tok, double eps,
                         uint16_t *x_bf16, void *stream) {
    if (!layers || n_layers < 1) return fail(DS4MOE_EINVAL, "forward_stack: no layers");
    if (n_tok < 0 || !(eps >= 0.0)) return fail(DS4MOE_EINVAL, "forward_stack: n_tok %d, eps %g", n_tok, eps);
    if (n_tok > 0 && (!h || !x_bf16)) return fail(DS4MOE_EINVAL, "forward_stack: NULL h or x");
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
    }
    if (n_tok == 0) return DS4MOE_OK;
    const int E = layers[0]->L.n_embd;
    for (int l = 0; l < n_layers; ++l) {
        hipError_t e = launch_rmsnorm(h, n_tok, E, eps, x_bf16, (hipStream_t)stream);
        if (e != hipSuccess) return fail(DS4MOE_EHIP, "forward_stack: layer %d rmsnorm: %s", l, hipGetErrorString(e));
        int rc = ds4moe_forward(layers[l], x_bf16, n_tok, h, stream);
        if (rc) return fail(rc, "forward_stack: layer %d: %s", l, g_err.c_str());
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
