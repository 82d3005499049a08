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


def cpu_baseline_decode(layer, x_np, budget_s=12.0):
    """The oracle (as it stands) on the host cores, on a bounded sample of the same
    token stream: batches of 16 tokens until about budget_s seconds have passed."""
    import oracle
    done, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(layer, x_np[done:done + 16])
        done += 16
        el = time.perf_counter() - t0
        if el >= budget_s or done + 16 > len(x_np):
            break
    return {"value": done / el, "unit": "tok/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"first {done} of the 1000 decode tokens, oracle.forward in batches of 16 "
                      f"({el:.1f} s)"}


def run_decode(args):
    import numpy as np
    import torch

    import bit_quantized_moe_renorm_amd as m
    from bit_quantized_moe_renorm_amd import synth

    spec = synth.DS4
    t0 = time.perf_counter()
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
    # duration is the timed region's events divided by the launches in it
    dom = max(per_kernel, key=lambda k: per_kernel[k]["bytes"])
    achieved = round(kb[dom] / (region_us * 1e-6) / 1e9, 1)
    traffic = profile_traffic("decode_b1_ds4_k_decode_fused.md") if dom == "fused" else None
    log(f"[bench] {dom}: {region_us:.2f} us per launch over the timed region (events), {achieved} GB/s algorithmic")

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
                     "algorithmic_bytes_per_launch": kb[dom], "avg_launch_us": round(region_us, 3)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(layer, x_np)
        log(f"[bench] cpu baseline: {res['cpu_baseline']}")
    for r in reps:
        r.close()
    return res


def flops_prefill(spec, n):
    """Algorithmic floating-point operations of each batched-path kernel for n tokens
    (2 per multiply-add; the Q2_K min term and the shared expert's low-part
    MFMAs are implementation overhead and not counted)."""
    E, F, NE, k = spec.n_embd, spec.n_ff, spec.n_expert, spec.top_k
    S = n * k
    return {"route": 2 * n * E * NE, "gemm_gateup_routed": 4 * E * F * S, "gemm_gateup_shared": 4 * E * F * n,
            "gemm_down_routed": 2 * E * F * S, "gemm_down_shared": 2 * E * F * n}


def run_prefill(args):
    import numpy as np
    import torch

    import bit_quantized_moe_renorm_amd as m
    from bit_quantized_moe_renorm_amd import synth

    spec = synth.DS4
    n = args.tokens
    layer = synth.make_layer(spec, seed=1)
    x_np = synth.activations(1, n, spec.n_embd)
    w = m.upload_layer(layer)
    dev = m.MoELayer(spec, w, max_tokens=n)
    del w
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    x = m.to_device_x(x_np)
    out = torch.zeros((n, spec.n_embd), dtype=torch.float32, device="cuda")
    for _ in range(args.warmup):
        dev.forward(x, out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dev.forward(x, out)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dev.timing_enable(True)
    for _ in range(args.steps):
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
        per_kernel[kind] = d
    log("[bench] prefill per-kernel: " + json.dumps(per_kernel))
    dom = "gemm_gateup_routed"
    achieved = per_kernel[dom]["TFLOP_s"]
    ms_step = 1000.0 * wall / args.steps
    tok_s = n / (wall / args.steps)
    total_tf = sum(fl.values()) / (wall / args.steps) / 1e12
    log(f"[bench] prefill {n}: {ms_step:.3f} ms/step, {tok_s:.0f} tok/s, {total_tf:.0f} TFLOP/s whole layer")
    res = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16/bf16 MFMA, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": f"DS4-shape MoE layer prefill of {n} tokens in one call (n_embd 4096, n_ff 2048, "
                               "256 experts, top-6, 1 shared; IQ2-style gate/up, Q2_K-style down; seed 1)",
                   "global_batch": n, "seq_len": n, "parallelism": "none (1 GPU)",
                   "layer_TFLOP_s": round(total_tf, 1), "layer_flop": sum(fl.values()),
                   "per_kernel": per_kernel},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None},
    }
    dev.close()
    return res


def run_stack(args):
    """The layer stack: L DS4-shape layers with seeds 4000 + l, each RMSNorm
    (unit gain, eps 1e-6) -> MoE block -> residual add on an fp32 stream.
    Decode: 256 steps of one token through all layers.  Prefill: 4096 tokens
    in 512-token chunks through all layers."""
    import torch

    import bit_quantized_moe_renorm_amd as m
    from bit_quantized_moe_renorm_amd import synth

    spec = synth.DS4
    L, chunk, n_pre, n_dec = args.layers, 512, 4096, 256
    devs = []
    t0 = time.perf_counter()
    for l in range(L):
        lay = synth.make_layer(spec, seed=4000 + l)
        w = m.upload_layer(lay)
        devs.append(m.MoELayer(spec, w, max_tokens=chunk))
        del w, lay
        torch.cuda.synchronize()
        log(f"[bench] stack: layer {l + 1}/{L} resident ({time.perf_counter() - t0:.0f} s)")
    torch.cuda.empty_cache()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # decode b = 1
    h = torch.from_numpy(synth.residual(41, n_dec + 8, spec.n_embd)).cuda()
    xb = torch.empty((1, spec.n_embd), dtype=torch.bfloat16, device="cuda")

    def token(t):
        m.forward_stack(devs, h[t:t + 1], x=xb, stream=stream)

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
    xp = torch.empty((chunk, spec.n_embd), dtype=torch.bfloat16, device="cuda")

    def prefill():
        for c0 in range(0, n_pre, chunk):
            m.forward_stack(devs, hp[c0:c0 + chunk], x=xp, stream=stream)

    prefill()                               # warm-up pass (the stream's values are not checked here)
    torch.cuda.synchronize()
    ev0.record(stream)
    prefill()
    ev1.record(stream)
    torch.cuda.synchronize()
    pre_s = ev0.elapsed_time(ev1) * 1e-3
    fl = sum(flops_prefill(spec, chunk).values()) * (n_pre // chunk) * L
    pre_tok_s = n_pre / pre_s
    log(f"[bench] stack of {L} prefill {n_pre} in {chunk}-token chunks: {pre_tok_s:.0f} tok/s, "
        f"{fl / pre_s / 1e12:.0f} TFLOP/s = {100 * fl / pre_s / 1e12 / BF16_PEAK_TFLOPS:.1f}% of bf16 peak")
    for dev in devs:
        dev.close()
    return {
        "metric": METRIC, "value": round(dec_tok_s, 2), "unit": "tok/s", "n_gpus": 1,
        "steps": n_dec, "warmup": 8, "ms_per_step": round(1e3 * dec_s / n_dec, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"stack of {L} DS4-shape MoE layers (seeds 4000..{4000 + L - 1}), RMSNorm -> MoE -> "
                               "residual add per layer, decode b=1 over 256 steps; prefill 4096 tokens in "
                               "512-token chunks",
                   "global_batch": 1, "seq_len": 1, "parallelism": "none (1 GPU)", "layers": L,
                   "decode_layer_us": round(1e6 * dec_s / n_dec / L, 3),
                   "decode_hbm_GB_s": round(dec_gbs, 1), "decode_hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                   "prefill_tok_s": round(pre_tok_s, 1), "prefill_TFLOP_s": round(fl / pre_s / 1e12, 1),
                   "prefill_mfma_frac": round(fl / pre_s / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "roofline": {"bound": "hbm", "kernel": "fused", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": None},
    }


def run_batch(args):
    """Small-batch decode (n = 8, 16, 32 tokens per call) of the DS4-shape layer
    under a Zipf(1.1)-biased router, 8 layer replicas cycled so the weights
    come from HBM.  Bytes per call: the distinct routed experts the call
    touches (counted from its own routing) times an expert's bytes, plus the
    shared expert and the router."""
    import numpy as np
    import torch

    import bit_quantized_moe_renorm_amd as m
    from bit_quantized_moe_renorm_amd import synth

    spec = synth.DS4
    lay = synth.make_layer(spec, seed=1, zipf_bias=True)
    devs = []
    for _ in range(args.replicas):
        w = m.upload_layer(lay)
        devs.append(m.MoELayer(spec, w, max_tokens=64))
        del w
    nb = synth.layer_nbytes(spec)
    router_bytes = spec.n_expert * spec.n_embd * 4
    steps = 200
    x = m.to_device_x(synth.activations(2, 32 * (steps + 8), spec.n_embd))
    out = torch.zeros((32, spec.n_embd), dtype=torch.float32, device="cuda")
    rows = {}
    for n in (8, 16, 32):
        # distinct experts per call, from the library's own routing of the same tokens
        uniq = []
        for it in range(steps):
            _, _, off, _ = devs[0].route(x[n * it:n * it + n])
            o = off.cpu().numpy()
            uniq.append(int(np.count_nonzero(o[1:] - o[:-1])))
        for it in range(8):
            devs[it % len(devs)].forward(x[n * it:n * it + n], out[:n])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for it in range(steps):
            devs[it % len(devs)].forward(x[n * it:n * it + n], out[:n])
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        u = float(np.mean(uniq))
        gbs = (u * nb["per_expert"] + nb["shared"] + router_bytes) / dt / 1e9
        rows[n] = {"us_per_call": round(dt * 1e6, 2), "tok_s": round(n / dt, 1), "distinct_experts": round(u, 2),
                   "GB_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        log(f"[bench] batch {n}: {dt * 1e6:.1f} us per call, {n / dt:.0f} tok/s, {u:.1f} distinct experts, "
            f"{gbs:.0f} GB/s = {100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s")
    for d in devs:
        d.close()
    r32 = rows[32]
    return {
        "metric": METRIC, "value": r32["tok_s"], "unit": "tok/s", "n_gpus": 1, "steps": steps, "warmup": 8,
        "ms_per_step": round(r32["us_per_call"] / 1000, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "DS4-shape MoE layer, small-batch decode of 8/16/32 tokens per call under a "
                               "Zipf(1.1) router bias (seed 1; value = 32 tokens)", "global_batch": 32,
                   "seq_len": 1, "parallelism": "none (1 GPU)", "replicas": args.replicas,
                   "per_batch": {str(k): v for k, v in rows.items()}},
        "roofline": {"bound": "hbm", "kernel": "whole call", "achieved": r32["GB_s"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": r32["hbm_frac"], "traffic": None},
    }


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
    ap.add_argument("--workload", choices=("decode", "prefill", "stack", "batch"), default="decode")
    ap.add_argument("--layers", type=int, default=43, help="stack workload: number of layers")
    ap.add_argument("--tokens", type=int, default=2048, help="prefill tokens per call")
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
        if args.steps == 1000 and args.warmup == 100:   # defaults sized for decode
            args.steps, args.warmup = 50, 5
        res = run_prefill(args)
    elif args.workload == "stack":
        res = run_stack(args)
    elif args.workload == "batch":
        res = run_batch(args)
    else:
        res = run_decode(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
