#!/usr/bin/env python3
"""Benchmark of the 2-bit routed-MoE block on one MI355X.

Default workload (a step = one decode token through one DS4-shape MoE layer:
router, top-6, bucketing, 6 routed IQ2/Q2_K experts, bf16 shared expert and
the weighted scatter into the residual):
  n_embd 4096, n_ff 2048, 256 experts, top-6, 1 shared expert, seed 1,
  a stream of 1000 seeded N(0,1) bf16 tokens, one forward call per token.

The layer is created R times (identical bytes, separate buffers) and the
steps cycle through the copies, so consecutive uses of one copy are R * 97 MB
apart and nothing is served from the 256 MB Infinity Cache: every step
streams its weights from HBM, as in a stack of distinct layers.

The default run also times the 2048-token prefill of the same layer (one
call, and four calls of 512 tokens), nested under "prefill" with its own MFMA
roofline and CPU baseline: the metric names both halves.

Prints ONE JSON line on stdout; details go to stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "MoE-layer tok/s + achieved HBM GB/s (% of peak), decode b=1 and prefill 2048"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def touched_bytes(spec, n_distinct_experts, shared=True):
    from bit_quantized_moe_renorm_amd import synth
    nb = synth.layer_nbytes(spec)
    return n_distinct_experts * nb["per_expert"] + (nb["shared"] if shared else 0)


def kernel_bytes_decode(spec):
    """Algorithmic bytes per launch of each decode kernel at b = 1 (6 distinct experts).

    "fused" is the single persistent launch that reads all of them: the router
    (fp32), the shared expert (bf16) and the 6 selected experts as stored."""
    from bit_quantized_moe_renorm_amd import synth
    nb = synth.layer_nbytes(spec)
    E, F, k = spec.n_embd, spec.n_ff, spec.top_k
    parts = {
        "route": nb["router"],
        "gateup_shared": 2 * E * F * 2,
        "gateup_routed": k * 2 * nb["gate"],
        "down_routed": k * nb["down"],
        "down_shared": E * F * 2,
    }
    parts["fused"] = sum(parts.values())
    return parts


def profile_traffic(name):
    """HBM bytes per launch of a kernel from its committed rocprofv3 counter
    summary under profiles/ (FETCH_SIZE and WRITE_SIZE, each scaled by what the
    counter reads for a copy of known size), or None if there is none or the
    kernel's sources changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", name)
    try:
        text = open(path).read()
    except OSError:
        return None
    tb = re.search(r"^traffic_bytes_per_launch: (\d+)$", text, re.M)
    srcs = re.search(r"^kernel_sources: (.+)$", text, re.M)
    sha = re.search(r"^kernel_source_sha256: ([0-9a-f]{64})$", text, re.M)
    if not (tb and srcs and sha):
        return None
    h = hashlib.sha256()
    for f in srcs.group(1).split():
        try:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        except OSError:
            return None
    return int(tb.group(1)) if h.hexdigest() == sha.group(1) else None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(fn, n_tok):
    t0 = time.perf_counter()
    fn()
    return n_tok / (time.perf_counter() - t0)


def cpu_baseline(fn_all, n_all, fn_one, n_one, unit, sample, sample_one):
    """The oracle (as it stands) on the host cores: fn_all covers n_all tokens
    with every OpenMP thread (or returns how many it covered, when n_all is
    None), fn_one n_one tokens with one thread."""
    import oracle
    cores = oracle.num_threads()
    t0 = time.perf_counter()
    r = fn_all()
    el = time.perf_counter() - t0
    if n_all is None:
        n_all = r
    oracle.set_num_threads(1)
    try:
        one = _oracle_rate(fn_one, n_one)
    finally:
        oracle.set_num_threads(cores)
    return {"value": round(n_all / el, 3), "unit": unit, "cores": cores, "kind": "oracle",
            "sample": f"{sample}: {n_all} tokens in {el:.1f} s", "cpu_model": cpu_model(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "one_thread": {"value": round(one, 3), "unit": unit, "sample": sample_one}}


def cpu_baseline_decode(layer, x_np, budget_s=12.0):
    """The oracle on a bounded sample of the decode token stream: batches of 16
    tokens until about budget_s seconds have passed."""
    import oracle

    def run():
        done, t0 = 0, time.perf_counter()
        while True:
            oracle.forward(layer, x_np[done:done + 16])
            done += 16
            if time.perf_counter() - t0 >= budget_s or done + 16 > len(x_np):
                return done

    return cpu_baseline(run, None, lambda: oracle.forward(layer, x_np[:1]), 1, "tok/s",
                        "the first tokens of the 1000-token decode stream, oracle.forward in batches of 16",
                        "token 0")


def run_decode(args, layer=None):
    import numpy as np
    import torch

    import bit_quantized_moe_renorm_amd as m
    from bit_quantized_moe_renorm_amd import synth

    spec = synth.DS4
    t0 = time.perf_counter()
    if layer is None:
        layer = synth.make_layer(spec, seed=1)
    x_np = synth.activations(1, 1000, spec.n_embd)
    log(f"[bench] generated layer + 1000 tokens in {time.perf_counter() - t0:.1f} s")
    w = m.upload_layer(layer)
    reps = [m.MoELayer(spec, w, max_tokens=1) for _ in range(args.replicas)]
    del w
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    x = m.to_device_x(x_np)
    out = torch.zeros((1000, spec.n_embd), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    R = len(reps)

    def step(i):
        t = i % 1000
        reps[i % R].forward(x[t:t + 1], out[t:t + 1], stream)

    for i in range(args.warmup):
        step(i)
    # pass 1 (the value): K steps back to back, bracketed by synchronisation;
    # HIP events on the launch stream around the same region give the fused
    # kernel's average duration (one launch per step, nothing else queued)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    region_us = 1000.0 * ev0.elapsed_time(ev1) / args.steps
    # pass 2 (kernel durations): the same K steps with HIP events recorded by the
    # library around each kernel on the caller's stream (an event pair per launch
    # adds about 4 us of stream time, so pass 1 alone gives the throughput)
    for r in reps:
        r.timing_enable(True)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + args.steps + i)
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t2
    tot = {}
    for r in reps:
        for kind, (ms, cnt) in r.timing_read().items():
            a = tot.setdefault(kind, [0.0, 0])
            a[0] += ms
            a[1] += cnt
        r.timing_enable(False)
    avg_us = {k: 1000.0 * v[0] / v[1] for k, v in tot.items() if v[1]}
    log(f"[bench] pass with per-launch events: {1e6 * wall_ev / args.steps:.2f} us/step")
    kb = kernel_bytes_decode(spec)
    per_kernel = {k: {"avg_us": round(avg_us[k], 3), "bytes": kb[k],
                      "GB_s": round(kb[k] / (avg_us[k] * 1e-6) / 1e9, 1)} for k in avg_us if k in kb}
    log("[bench] per-kernel: " + json.dumps(per_kernel))
    # the kernel with the most algorithmic bytes is the dominant one; its
    # duration is the timed region's events divided by the launches in it.
    # Algorithmic bytes: the touched expert bytes as stored (6 routed experts +
    # the shared expert); the router's 4 MB counts in time, not in bytes.
    dom = max(per_kernel, key=lambda k: per_kernel[k]["bytes"])
    alg_bytes = touched_bytes(spec, spec.top_k) if dom == "fused" else kb[dom]
    achieved = round(alg_bytes / (region_us * 1e-6) / 1e9, 1)
    achieved_router = round(kb[dom] / (region_us * 1e-6) / 1e9, 1)
    traffic = profile_traffic("decode_b1_ds4_k_decode_fused.md") if dom == "fused" else None
    log(f"[bench] {dom}: {region_us:.2f} us per launch over the timed region (events), {achieved} GB/s "
        f"algorithmic ({achieved_router} GB/s counting the router's bytes too)")

    tok_s = args.steps / wall
    ms_step = 1000.0 * wall / args.steps
    layer_bytes = touched_bytes(spec, spec.top_k)
    layer_gbs = layer_bytes / (wall / args.steps) / 1e9
    log(f"[bench] decode b=1: {tok_s:.0f} tok/s, {ms_step * 1000:.2f} us/token, touched-expert "
        f"{layer_gbs:.0f} GB/s = {100 * layer_gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s")

    res = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "DS4-shape MoE layer decode b=1 (n_embd 4096, n_ff 2048, 256 experts, top-6, "
                               "1 shared; IQ2-style gate/up, Q2_K-style down; seed 1; 1000-token stream)",
                   "global_batch": 1, "seq_len": 1, "parallelism": "none (1 GPU)",
                   "replicas": R,
                   "touched_expert_bytes_per_token": layer_bytes,
                   "layer_GB_s": round(layer_gbs, 1),
                   "layer_hbm_frac": round(layer_gbs / HBM_PEAK_GBS, 4),
                   "per_kernel": per_kernel},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "traffic_unit": "bytes per launch",
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "bytes_per_launch_with_router": kb[dom], "achieved_with_router": achieved_router,
                     "frac_with_router": round(achieved_router / HBM_PEAK_GBS, 4),
                     "avg_launch_us": round(region_us, 3)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(layer, x_np)
        log(f"[bench] cpu baseline: {res['cpu_baseline']}")
    for r in reps:
        r.close()
    return res


def run_decode_hash(args, layer):
    """The same decode stream through a hash-routed layer (the experts of each
    token from its id's table row): the block's time when only the k table
    experts' router rows are read.  Token ids: the seed's uniform id stream."""
    import torch

    import bit_quantized_moe_renorm_amd as m
    from bit_quantized_moe_renorm_amd import synth

    spec = synth.DS4
    lay = synth.Layer(**{**layer.__dict__})
    lay.hash_table = synth.hash_table(1, synth.N_VOCAB, spec.n_expert, spec.top_k)
    w = m.upload_layer(lay)
    reps = [m.MoELayer(spec, w, max_tokens=1) for _ in range(args.replicas)]
    del w
    x = m.to_device_x(synth.activations(1, 1000, spec.n_embd))
    ids = m.to_device_ids(synth.token_ids(1, 1000))
    out = torch.zeros((1000, spec.n_embd), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    R = len(reps)

    def step(i):
        t = i % 1000
        reps[i % R].forward(x[t:t + 1], out[t:t + 1], stream, ids=ids[t:t + 1])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for r in reps:
        assert r.status() == m.OK
        r.close()
    us = 1e6 * wall / args.steps
    gbs = touched_bytes(spec, spec.top_k) / (wall / args.steps) / 1e9
    log(f"[bench] hash-routed layer decode b=1: {args.steps / wall:.0f} tok/s, {us:.2f} us/token, "
        f"touched-expert {gbs:.0f} GB/s = {100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s")
    return {"value": round(args.steps / wall, 1), "unit": "tok/s", "us_per_token": round(us, 3),
            "steps": args.steps, "warmup": args.warmup,
            "workload": "the decode stream above through a hash-routed layer (same weights; table of "
                        f"{synth.N_VOCAB} x {spec.top_k} experts, seed 1; token ids uniform, seed 1)",
            "layer_GB_s": round(gbs, 1), "layer_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "router_bytes_read": spec.top_k * spec.n_embd * 4}


def flops_prefill(spec, n):
    """Algorithmic floating-point operations of each batched-path kernel for n tokens
    (2 per multiply-add; the Q2_K min term and the shared expert's low-part
    MFMAs are implementation overhead and not counted)."""
    E, F, NE, k = spec.n_embd, spec.n_ff, spec.n_expert, spec.top_k
    S = n * k
    return {"route": 2 * n * E * NE, "gemm_gateup_routed": 4 * E * F * S, "gemm_gateup_shared": 4 * E * F * n,
            "gemm_down_routed": 2 * E * F * S, "gemm_down_shared": 2 * E * F * n}


def layer_flop(spec, n):
    """Routed (selected) + shared matmul flops of a layer for n tokens; the
    router's flops count in time, not in the numerator."""
    fl = flops_prefill(spec, n)
    return sum(v for k, v in fl.items() if k != "route")


def distinct_experts(off):
    import numpy as np
    o = off.cpu().numpy()
    return int(np.count_nonzero(o[1:] - o[:-1]))


def run_prefill(args, layer=None, cpu=True):
    """The 2048-token prefill of the DS4-shape layer (seed 1 weights, seed 1
    tokens): one call of 2048 tokens (MFMA-bound; roofline against the bf16
    peak) and the same tokens in four calls of 512 (HBM-bound: every call
    streams nearly all 256 experts; reported against the HBM peak)."""
    import numpy as np
    import torch

    import bit_quantized_moe_renorm_amd as m
    from bit_quantized_moe_renorm_amd import synth

    spec = synth.DS4
    n = args.tokens
    steps, warmup = args.prefill_steps, args.prefill_warmup
    if layer is None:
        layer = synth.make_layer(spec, seed=1)
    x_np = synth.activations(1, n, spec.n_embd)
    w = m.upload_layer(layer)
    dev = m.MoELayer(spec, w, max_tokens=n)
    del w
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    x = m.to_device_x(x_np)
    out = torch.zeros((n, spec.n_embd), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        dev.forward(x, out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dev.forward(x, out)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    u_one = distinct_experts(dev.last_routing(n)[2])
    dev.timing_enable(True)
    for _ in range(steps):
        dev.forward(x, out)
    torch.cuda.synchronize()
    tim = dev.timing_read()
    dev.timing_enable(False)
    fl = flops_prefill(spec, n)
    per_kernel = {}
    for kind, (ms, cnt) in tim.items():
        us = 1000.0 * ms / cnt
        d = {"avg_us": round(us, 2)}
        if kind in fl:
            d["TFLOP_s"] = round(fl[kind] / (us * 1e-6) / 1e12, 1)
            if kind != "route":
                d["mfma_frac"] = round(fl[kind] / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)
        per_kernel[kind] = d
    log("[bench] prefill per-kernel: " + json.dumps(per_kernel))
    dom = "gemm_gateup_routed"
    achieved = per_kernel[dom]["TFLOP_s"]
    step_s = wall / steps
    tok_s = n / step_s
    lf = layer_flop(spec, n)
    layer_tf = lf / step_s / 1e12
    nb = synth.layer_nbytes(spec)
    bytes_one = u_one * nb["per_expert"] + nb["shared"]
    log(f"[bench] prefill {n}: {1000 * step_s:.3f} ms/step, {tok_s:.0f} tok/s, {layer_tf:.0f} TFLOP/s whole layer "
        f"= {100 * layer_tf / BF16_PEAK_TFLOPS:.1f}% of bf16 peak; {dom} {achieved} TFLOP/s")

    # the same tokens in calls of 512: memory-bound
    chunk = 512
    devc = m.MoELayer(spec, m.upload_layer(layer), max_tokens=chunk)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    outc = torch.zeros_like(out)

    def chunked():
        for c0 in range(0, n, chunk):
            devc.forward(x[c0:c0 + chunk], outc[c0:c0 + chunk])

    for _ in range(warmup):
        chunked()
    us = []
    for c0 in range(0, n, chunk):
        devc.forward(x[c0:c0 + chunk], outc[c0:c0 + chunk])
        us.append(distinct_experts(devc.last_routing(chunk)[2]))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        chunked()
    torch.cuda.synchronize()
    wall_c = time.perf_counter() - t0
    call_s = wall_c / steps / (n // chunk)
    bytes_c = float(np.mean(us)) * nb["per_expert"] + nb["shared"]
    gbs_c = bytes_c / call_s / 1e9
    tf_c = layer_flop(spec, chunk) / call_s / 1e12
    log(f"[bench] prefill {n} in {chunk}-token calls: {1e6 * call_s:.1f} us per call, {chunk / call_s:.0f} tok/s, "
        f"{float(np.mean(us)):.1f} experts touched, {gbs_c:.0f} GB/s = {100 * gbs_c / HBM_PEAK_GBS:.1f}% of 8 TB/s, "
        f"{tf_c:.0f} TFLOP/s")
    devc.close()

    res = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tok/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(1000 * step_s, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16/fp16 MFMA, fp32 accumulate", "data": "synthetic",
        "config": {"workload": f"DS4-shape MoE layer prefill of {n} tokens in one call (n_embd 4096, n_ff 2048, "
                               "256 experts, top-6, 1 shared; IQ2-style gate/up, Q2_K-style down; seed 1)",
                   "global_batch": n, "seq_len": n, "parallelism": "none (1 GPU)",
                   "layer_TFLOP_s": round(layer_tf, 1), "layer_flop": lf,
                   "layer_mfma_frac": round(layer_tf / BF16_PEAK_TFLOPS, 4),
                   "distinct_experts": u_one, "touched_expert_bytes": bytes_one,
                   "layer_hbm_frac": round(bytes_one / step_s / 1e9 / HBM_PEAK_GBS, 4),
                   "per_kernel": per_kernel},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "traffic": profile_traffic("prefill_2048_ds4_gemm_kernels.md"),
                     "traffic_unit": "bytes per launch",
                     "algorithmic_flop_per_launch": fl[dom], "avg_launch_us": per_kernel[dom]["avg_us"]},
        "chunks_512": {"us_per_call": round(1e6 * call_s, 2), "tok_s": round(chunk / call_s, 1),
                       "distinct_experts": round(float(np.mean(us)), 2), "touched_expert_bytes": round(bytes_c),
                       "GB_s": round(gbs_c, 1), "hbm_frac": round(gbs_c / HBM_PEAK_GBS, 4),
                       "TFLOP_s": round(tf_c, 1), "mfma_frac": round(tf_c / BF16_PEAK_TFLOPS, 4)},
    }
    if cpu:
        import oracle
        ns = args.prefill_cpu_tokens
        res["cpu_baseline"] = cpu_baseline(
            lambda: oracle.forward(layer, x_np[:ns]), ns, lambda: oracle.forward(layer, x_np[:4]), 4, "tok/s",
            f"oracle.forward on the first {ns} of the {n} prefill tokens in one call", "first 4 prefill tokens")
        log(f"[bench] prefill cpu baseline: {res['cpu_baseline']}")
    dev.close()
    return res


def run_stack(args):
    """The layer stack: L DS4-shape layers with seeds 4000 + l, each RMSNorm
    (unit gain, eps 1e-6) -> MoE block -> residual add on an fp32 stream.
    Decode: 256 steps of one token through all layers.  Prefill: 4096 tokens
    in 512-token chunks through all layers.  After the timed runs, a
    teacher-forced check: a few decode tokens run layer by layer, and for
    every layer the oracle takes the GPU's own x_l and recomputes the routing
    and the block output; its time is the CPU baseline."""
    import numpy as np
    import torch

    import bit_quantized_moe_renorm_amd as m
    from bit_quantized_moe_renorm_amd import synth

    spec = synth.DS4
    L, chunk, n_pre, n_dec = args.layers, 512, 4096, 256
    n_hash = min(args.hash_layers, L)
    devs, hosts = [], []
    t0 = time.perf_counter()
    for l in range(L):
        lay = synth.make_layer(spec, seed=4000 + l)
        if l < n_hash:
            lay.hash_table = synth.hash_table(4000 + l, synth.N_VOCAB, spec.n_expert, spec.top_k)
        w = m.upload_layer(lay)
        devs.append(m.MoELayer(spec, w, max_tokens=chunk))
        hosts.append(lay if not args.no_cpu_baseline else None)
        del w, lay
        torch.cuda.synchronize()
        log(f"[bench] stack: layer {l + 1}/{L} resident ({time.perf_counter() - t0:.0f} s)")
    torch.cuda.empty_cache()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # decode b = 1
    h = torch.from_numpy(synth.residual(41, n_dec + 8, spec.n_embd)).cuda()
    ids_dec = m.to_device_ids(synth.token_ids(41, n_dec + 8))
    xb = torch.empty((1, spec.n_embd), dtype=torch.bfloat16, device="cuda")

    def token(t):
        m.forward_stack(devs, h[t:t + 1], x=xb, stream=stream, ids=ids_dec[t:t + 1])

    for t in range(8):                      # warm-up tokens
        token(n_dec + t)
    torch.cuda.synchronize()
    ev0.record(stream)
    for t in range(n_dec):
        token(t)
    ev1.record(stream)
    torch.cuda.synchronize()
    dec_s = ev0.elapsed_time(ev1) * 1e-3
    dec_tok_s = n_dec / dec_s
    layer_bytes = touched_bytes(spec, spec.top_k)
    dec_gbs = L * layer_bytes * n_dec / dec_s / 1e9
    log(f"[bench] stack of {L} decode b=1: {dec_tok_s:.1f} tok/s, {1e6 * dec_s / n_dec / L:.2f} us per layer-token, "
        f"{dec_gbs:.0f} GB/s touched-expert bytes = {100 * dec_gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s")

    # prefill: 4096 tokens in 512-token chunks
    hp = torch.from_numpy(synth.residual(42, n_pre, spec.n_embd)).cuda()
    ids_pre = m.to_device_ids(synth.token_ids(42, n_pre))
    xp = torch.empty((chunk, spec.n_embd), dtype=torch.bfloat16, device="cuda")

    def prefill():
        for c0 in range(0, n_pre, chunk):
            m.forward_stack(devs, hp[c0:c0 + chunk], x=xp, stream=stream, ids=ids_pre[c0:c0 + chunk])

    prefill()                               # warm-up pass (the stream's values are not checked here)
    torch.cuda.synchronize()
    ev0.record(stream)
    prefill()
    ev1.record(stream)
    torch.cuda.synchronize()
    pre_s = ev0.elapsed_time(ev1) * 1e-3
    fl = layer_flop(spec, chunk) * (n_pre // chunk) * L
    pre_tok_s = n_pre / pre_s
    nb = synth.layer_nbytes(spec)
    pre_bytes = L * (n_pre // chunk) * (spec.n_expert * nb["per_expert"] + nb["shared"])
    log(f"[bench] stack of {L} prefill {n_pre} in {chunk}-token chunks: {pre_tok_s:.0f} tok/s, "
        f"{fl / pre_s / 1e12:.0f} TFLOP/s = {100 * fl / pre_s / 1e12 / BF16_PEAK_TFLOPS:.1f}% of bf16 peak, "
        f"{pre_bytes / pre_s / 1e9:.0f} GB/s = {100 * pre_bytes / pre_s / 1e9 / HBM_PEAK_GBS:.1f}% of 8 TB/s")

    res = {
        "metric": METRIC, "value": round(dec_tok_s, 2), "unit": "tok/s", "n_gpus": 1,
        "steps": n_dec, "warmup": 8, "ms_per_step": round(1e3 * dec_s / n_dec, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"stack of {L} DS4-shape MoE layers (seeds 4000..{4000 + L - 1}; the first "
                               f"{n_hash} hash-routed by token id), RMSNorm -> MoE -> "
                               "residual add per layer, decode b=1 over 256 steps; prefill 4096 tokens in "
                               "512-token chunks",
                   "hash_layers": n_hash,
                   "global_batch": 1, "seq_len": 1, "parallelism": "none (1 GPU)", "layers": L,
                   "decode_layer_us": round(1e6 * dec_s / n_dec / L, 3),
                   "decode_hbm_GB_s": round(dec_gbs, 1), "decode_hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                   "prefill_tok_s": round(pre_tok_s, 1), "prefill_TFLOP_s": round(fl / pre_s / 1e12, 1),
                   "prefill_mfma_frac": round(fl / pre_s / 1e12 / BF16_PEAK_TFLOPS, 4),
                   "prefill_hbm_GB_s": round(pre_bytes / pre_s / 1e9, 1),
                   "prefill_hbm_frac": round(pre_bytes / pre_s / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "kernel": "fused (decode, all layers)", "achieved": round(dec_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None},
    }
    if not args.no_cpu_baseline:
        import oracle
        # teacher-forced: n_chk decode tokens layer by layer on the GPU, keeping
        # every layer's x_l, block output and routing; the oracle recomputes
        # each layer from the GPU's own x_l (its time is the CPU baseline)
        n_chk = args.stack_check_tokens
        hc = torch.from_numpy(synth.residual(45, n_chk, spec.n_embd)).cuda()
        ids_np = synth.token_ids(45, n_chk)
        ids_chk = m.to_device_ids(ids_np)
        rec = []
        for l, dev in enumerate(devs):
            xs = m.rmsnorm(hc)
            y = torch.zeros_like(hc)
            idx = []
            for t in range(n_chk):
                dev.forward(xs[t:t + 1], y[t:t + 1], ids=ids_chk[t:t + 1])
                idx.append(dev.last_routing(1)[0])
            torch.cuda.synchronize()
            rec.append((xs.view(torch.int16).cpu().numpy().view(np.uint16), y.cpu().numpy(),
                        torch.cat(idx).cpu().numpy()))
            hc = hc + y
        worst, same = 0.0, 0

        def check():
            nonlocal worst, same
            for l, (xl, yl, il) in enumerate(rec):
                ref, ridx, _ = oracle.forward(hosts[l], xl, token_ids=ids_np)
                d = np.max(np.abs(yl - ref)) / np.max(np.abs(ref))
                worst = max(worst, float(d))
                same += int(np.count_nonzero(np.all(il == ridx, axis=1)))

        res["cpu_baseline"] = cpu_baseline(
            check, n_chk, lambda: oracle.forward(hosts[-1], rec[-1][0][:1]), 1.0 / L, "tok/s",
            f"oracle.forward on {n_chk} decode tokens through all {L} layers, teacher-forced on the GPU's x_l",
            "one token through the last layer (tok/s through the whole stack = this / layers)")
        res["config"]["teacher_forced_check"] = {
            "tokens": n_chk, "layers": L, "routing_equal": f"{same}/{n_chk * L}",
            "max_rel_err_block_output": worst, "tolerance": 2e-3}
        log(f"[bench] stack teacher-forced check: routing equal {same}/{n_chk * L}, worst block-output rel err "
            f"{worst:.3e}; cpu baseline {res['cpu_baseline']}")
    for dev in devs:
        dev.close()
    return res


def run_batch(args):
    """Small-batch decode (n = 2, 7, 8, 16, 32 tokens per call; 2 and 7 are
    speculative verification shapes, the last token plus k = 1 or 6 drafted
    ones) of the DS4-shape layer under a Zipf(1.1)-biased router, 8 layer
    replicas cycled so the weights come from HBM.  Bytes per call: the
    distinct routed experts the call touches (counted from its own routing)
    times an expert's bytes, plus the shared expert."""
    import numpy as np
    import torch

    import bit_quantized_moe_renorm_amd as m
    import oracle
    from bit_quantized_moe_renorm_amd import synth

    spec = synth.DS4
    lay = synth.make_layer(spec, seed=1, zipf_bias=True)
    devs = []
    for _ in range(args.replicas):
        w = m.upload_layer(lay)
        devs.append(m.MoELayer(spec, w, max_tokens=64))
        del w
    nb = synth.layer_nbytes(spec)
    steps = 200
    x_np = synth.activations(2, 32 * (steps + 8), spec.n_embd)
    x = m.to_device_x(x_np)
    out = torch.zeros((32, spec.n_embd), dtype=torch.float32, device="cuda")
    rows = {}
    for n in (2, 7, 8, 16, 32):
        # distinct experts per call, from the library's own routing of the same tokens
        uniq = []
        for it in range(steps):
            _, _, off, _ = devs[0].route(x[n * it:n * it + n])
            uniq.append(distinct_experts(off))
        for it in range(8):
            devs[it % len(devs)].forward(x[n * it:n * it + n], out[:n])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for it in range(steps):
            devs[it % len(devs)].forward(x[n * it:n * it + n], out[:n])
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        u = float(np.mean(uniq))
        gbs = (u * nb["per_expert"] + nb["shared"]) / dt / 1e9
        row = {"us_per_call": round(dt * 1e6, 2), "tok_s": round(n / dt, 1), "distinct_experts": round(u, 2),
               "GB_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        if not args.no_cpu_baseline:
            row["cpu_baseline"] = cpu_baseline(
                lambda: oracle.forward(lay, x_np[:n]), n, lambda: oracle.forward(lay, x_np[:1]), 1, "tok/s",
                f"oracle.forward on one call of {n} tokens (the first of the stream)", "one token")
        rows[n] = row
        log(f"[bench] batch {n}: {dt * 1e6:.1f} us per call, {n / dt:.0f} tok/s, {u:.1f} distinct experts, "
            f"{gbs:.0f} GB/s = {100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s")
    for d in devs:
        d.close()
    r32 = rows[32]
    res = {
        "metric": METRIC, "value": r32["tok_s"], "unit": "tok/s", "n_gpus": 1, "steps": steps, "warmup": 8,
        "ms_per_step": round(r32["us_per_call"] / 1000, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "DS4-shape MoE layer, small-batch decode of 2/7/8/16/32 tokens per call under a "
                               "Zipf(1.1) router bias (seed 1; value = 32 tokens; 2 and 7 = MTP verification "
                               "of k = 1 and 6 drafts)", "global_batch": 32,
                   "seq_len": 1, "parallelism": "none (1 GPU)", "replicas": args.replicas,
                   "per_batch": {str(k): v for k, v in rows.items()}},
        "roofline": {"bound": "hbm", "kernel": "whole call", "achieved": r32["GB_s"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": r32["hbm_frac"], "traffic": None},
    }
    if "cpu_baseline" in r32:
        res["cpu_baseline"] = r32["cpu_baseline"]
    return res


def run_q4(args):
    """Decode b = 1 through a DS4-shape layer whose routed experts are
    Q4_K-style (the q4 model's format, 14.2 MB per expert): one forward call
    per token (router, then the dequant-fused GEMV kernels), replicas cycled
    so the weights come from HBM.  Bytes: 6 touched experts + the shared
    expert, as stored."""
    import torch

    import bit_quantized_moe_renorm_amd as m
    import oracle
    from bit_quantized_moe_renorm_amd import synth

    spec = synth.DS4
    lay = synth.make_layer(spec, seed=1, fmt="q4")
    x_np = synth.activations(1, 1000, spec.n_embd)
    w = m.upload_layer(lay)
    R = max(1, min(args.replicas, 8))
    reps = [m.MoELayer(spec, w, max_tokens=4) for _ in range(R)]
    del w
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    x = m.to_device_x(x_np)
    out = torch.zeros((1000, spec.n_embd), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    steps = min(args.steps, 1000)

    def step(i):
        t = i % 1000
        reps[i % R].forward(x[t:t + 1], out[t:t + 1], stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for r in reps:
        r.timing_enable(True)
    for i in range(steps):
        step(args.warmup + steps + i)
    torch.cuda.synchronize()
    tot = {}
    for r in reps:
        for kind, (ms, cnt) in r.timing_read().items():
            a = tot.setdefault(kind, [0.0, 0])
            a[0] += ms
            a[1] += cnt
        r.timing_enable(False)
    nb = synth.layer_nbytes(spec, "q4")
    E, F, k = spec.n_embd, spec.n_ff, spec.top_k
    kbytes = {"route": nb["router"], "gateup_shared": 2 * E * F * 2, "q4_gateup_routed": k * 2 * nb["gate"],
              "q4_down_routed": k * nb["down"], "down_shared": E * F * 2}
    per_kernel = {}
    for kind, (ms, cnt) in tot.items():
        us = 1000.0 * ms / cnt
        d = {"avg_us": round(us, 3)}
        if kind in kbytes:
            d["bytes"] = kbytes[kind]
            d["GB_s"] = round(kbytes[kind] / (us * 1e-6) / 1e9, 1)
        per_kernel[kind] = d
    log("[bench] q4 per-kernel: " + json.dumps(per_kernel))
    layer_bytes = k * nb["per_expert"] + nb["shared"]
    step_s = wall / steps
    gbs = layer_bytes / step_s / 1e9
    dom = "q4_gateup_routed"
    log(f"[bench] q4 decode b=1: {1e6 * step_s:.2f} us/token, {1 / step_s:.0f} tok/s, {gbs:.0f} GB/s touched "
        f"= {100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s")
    res = {
        "metric": METRIC, "value": round(1 / step_s, 1), "unit": "tok/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(1000 * step_s, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "DS4-shape MoE layer with Q4_K-style routed experts (q4 model), decode b=1, "
                               "seed 1, 1000-token stream", "global_batch": 1, "seq_len": 1,
                   "parallelism": "none (1 GPU)", "replicas": R, "touched_expert_bytes_per_token": layer_bytes,
                   "layer_GB_s": round(gbs, 1), "layer_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                   "per_kernel": per_kernel},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": per_kernel[dom]["GB_s"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(per_kernel[dom]["GB_s"] / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": kbytes[dom], "avg_launch_us": per_kernel[dom]["avg_us"]},
    }
    if not args.no_cpu_baseline:
        def run():
            done, t1 = 0, time.perf_counter()
            while time.perf_counter() - t1 < 10.0 and done + 4 <= 1000:
                oracle.forward(lay, x_np[done:done + 4])
                done += 4
            return done
        res["cpu_baseline"] = cpu_baseline(run, None, lambda: oracle.forward(lay, x_np[:1]), 1, "tok/s",
                                           "the first tokens of the decode stream, oracle.forward in batches of 4",
                                           "token 0")
    for r in reps:
        r.close()
    return res


def run_cache(args):
    """Decode b=1 through a DS4-shape layer whose routed experts live in pinned
    host memory, with an HBM cache of --cache-slots experts.  The router carries
    the Zipf(1.1) bias of the batch workload, so consecutive tokens reuse
    experts as a skewed real router would; without it every token would draw
    6 of 256 experts uniformly.  Each step: router, cache update, copy of the
    missed experts over the host link, the GEMV expert kernels."""
    import numpy as np
    import torch

    import bit_quantized_moe_renorm_amd as m
    from bit_quantized_moe_renorm_amd import synth

    spec = synth.DS4
    S = args.cache_slots
    layer = synth.make_layer(spec, seed=1)
    layer.router_bias = synth.zipf_router_bias(1, spec.n_expert)
    x_np = synth.activations(1, 1000, spec.n_embd)
    dev = m.MoELayer(spec, m.upload_layer(layer), max_tokens=1, cache_slots=S)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    x = m.to_device_x(x_np)
    out = torch.zeros((1000, spec.n_embd), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    steps = min(args.steps, 1000)

    def step(i):
        t = i % 1000
        dev.forward(x[t:t + 1], out[t:t + 1], stream)

    for i in range(args.warmup):
        step(i)
    s0 = dev.cache_stats()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    s1 = dev.cache_stats()
    # per-kernel pass (the cache kinds: update + copy)
    dev.timing_enable(True)
    s2 = dev.cache_stats()
    for i in range(steps):
        step(args.warmup + steps + i)
    torch.cuda.synchronize()
    tim = dev.timing_read()
    s3 = dev.cache_stats()
    dev.timing_enable(False)
    per_kernel = {k: round(1000.0 * ms / c, 3) for k, (ms, c) in tim.items()}
    # the host link's own rate: a 1 GiB copy from pinned host memory (the DMA
    # engines), the best of three
    src = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    link = 0.0
    for _ in range(3):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        dst.copy_(src, non_blocking=True)
        ev1.record(stream)
        torch.cuda.synchronize()
        link = max(link, (1 << 30) / (ev0.elapsed_time(ev1) * 1e-3) / 1e9)
    del src, dst
    hits, misses = s1["hits"] - s0["hits"], s1["misses"] - s0["misses"]
    host_bytes = s1["bytes"] - s0["bytes"]
    copy_ms = tim["cache"][0]
    copy_gbs = (s3["bytes"] - s2["bytes"]) / (copy_ms * 1e-3) / 1e9 if copy_ms > 0 else 0.0
    tok_s = steps / wall
    log(f"[bench] cache {S} slots decode b=1: {tok_s:.0f} tok/s, {1e6 * wall / steps:.1f} us/token, hit rate "
        f"{hits / max(1, hits + misses):.3f}, {host_bytes / steps / 1e6:.1f} MB/token from host, cache update + copy "
        f"at {copy_gbs:.1f} GB/s (host link by a pinned 1 GiB copy: {link:.1f} GB/s); per kernel (us): {per_kernel}")
    res = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tok/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(1000 * wall / steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"DS4-shape layer decode b=1 with host-resident routed experts and an HBM cache of "
                               f"{S} experts (Zipf(1.1)-biased router, seed 1; 1000-token stream)",
                   "global_batch": 1, "seq_len": 1, "parallelism": "none (1 GPU)", "cache_slots": S,
                   "hit_rate": round(hits / max(1, hits + misses), 4),
                   "misses_per_token": round(misses / steps, 3),
                   "host_bytes_per_token": round(host_bytes / steps),
                   "host_GB_s": round(host_bytes / wall / 1e9, 2),
                   "per_kernel_us": per_kernel},
        "roofline": {"bound": "host-link", "kernel": "cache update + copy", "achieved": round(copy_gbs, 2),
                     "peak": round(link, 2), "unit": "GB/s", "frac": round(copy_gbs / link, 4), "traffic": None,
                     "note": "bytes copied from pinned host memory per unit of the cache kernels' time; peak: the "
                             "rate of a 1 GiB pinned host-to-device copy measured in the same run"},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(layer, x_np)
    dev.close()
    return res


def copy_probe():
    """A plain device copy of known size, for calibrating the HBM byte counters
    (FETCH_SIZE / WRITE_SIZE) that the profiles of the block's kernels use."""
    import torch
    n = 64 << 20                      # 64 Mi fp32 = 256 MiB each way
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": 4 * n, "launches": 5}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="decode only (skip the nested prefill)")
    ap.add_argument("--no-hash-decode", action="store_true",
                    help="skip the hash-routed layer's decode figure (its launches are the same kernel)")
    ap.add_argument("--workload", choices=("decode", "prefill", "stack", "batch", "q4", "cache"), default="decode")
    ap.add_argument("--cache-slots", type=int, default=64, help="cache workload: HBM expert slots")
    ap.add_argument("--layers", type=int, default=43, help="stack workload: number of layers")
    ap.add_argument("--hash-layers", type=int, default=3,
                    help="stack workload: the first layers that are hash-routed (the model has 3)")
    ap.add_argument("--tokens", type=int, default=2048, help="prefill tokens per call")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--prefill-warmup", type=int, default=3)
    ap.add_argument("--prefill-cpu-tokens", type=int, default=256,
                    help="prefill tokens the oracle runs for the CPU baseline")
    ap.add_argument("--stack-check-tokens", type=int, default=2,
                    help="decode tokens of the stack's teacher-forced check (and CPU baseline)")
    ap.add_argument("--copy-probe", action="store_true", help="only run the counter-calibration copy")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X only: this build runs the MoE block on a single GPU "
              "(no multi-GPU path); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe()
        return
    if args.workload == "prefill":
        res = run_prefill(args, cpu=not args.no_cpu_baseline)
    elif args.workload == "stack":
        res = run_stack(args)
    elif args.workload == "batch":
        res = run_batch(args)
    elif args.workload == "q4":
        res = run_q4(args)
    elif args.workload == "cache":
        res = run_cache(args)
    else:
        from bit_quantized_moe_renorm_amd import synth
        layer = synth.make_layer(synth.DS4, seed=1)
        res = run_decode(args, layer)
        if not args.no_hash_decode:
            res["hash_layer_decode"] = run_decode_hash(args, layer)
        if not args.no_prefill:
            pre = run_prefill(args, layer, cpu=not args.no_cpu_baseline)
            res["prefill"] = {k: pre[k] for k in ("value", "unit", "ms_per_step", "steps", "warmup", "dtype",
                                                  "config", "roofline", "chunks_512", "cpu_baseline") if k in pre}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
