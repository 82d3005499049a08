"""Shared helpers for the GPU parity tests: cached layers, device uploads and
the comparison metrics.  Inputs come from the seeded generator only."""
import functools
import sys

import numpy as np

from bit_quantized_moe_renorm_amd import synth

# Output tolerance: max|gpu - ref| / max|ref| (the bar for every config).
REL_TOL = 2e-3
# The GEMV path keeps fp32 activations and exact weights; its error is
# a few fp32 roundings per dot product, far below the bar.  A tighter check
# catches wiring mistakes the loose bar would let through.
GEMV_TOL = 1e-5
# The fused single-token decode rounds each routed SwiGLU output h to fp16
# (11-bit significand, under a power-of-two scale per 64-value chunk that puts
# the chunk's largest value at the top of fp16's range) before the Q2_K down
# projections.  The rounding error of one h is at most 2^-12 of |h|; over the
# 2048 terms of a down row they add up like a random walk, to about
# 2^-12 / sqrt(3) ~ 1.4e-4 of the rms term, ~5e-5 of max|out| on the DS4 shapes.
# The check takes 4x that.
FUSED_TOL = 2e-4


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(gpu, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(gpu, np.float64) - ref)) / np.max(np.abs(ref)))


@functools.lru_cache(maxsize=None)
def host_layer(kind: str):
    if kind == "tiny":
        return synth.make_layer(synth.TINY, seed=0)
    if kind == "ds4":
        return synth.make_layer(synth.DS4, seed=1)
    if kind == "ds4_ties":
        # pairs of identical router rows (2j, 2j+1): every logit has an exact twin
        base = host_layer("ds4")
        lay = synth.Layer(**{**base.__dict__})
        r = base.router.copy()
        r[1::2] = r[0::2]
        lay.router = r
        return lay
    if kind == "ds4_zipf":
        base = host_layer("ds4")
        lay = synth.Layer(**{**base.__dict__})
        lay.router_bias = synth.zipf_router_bias(1, 256)
        return lay
    raise KeyError(kind)


_dev = {}


def device_layer(kind: str, max_tokens: int = 64):
    """A MoELayer handle (cached per kind and max_tokens)."""
    import bit_quantized_moe_renorm_amd as m
    key = (kind, max_tokens)
    if key not in _dev:
        lay = host_layer(kind)
        log(f"[gpu] create layer {kind} max_tokens={max_tokens}")
        w = m.upload_layer(lay)
        act = m.F32 if kind == "tiny" else m.BF16
        _dev[key] = m.MoELayer(lay.spec, w, max_tokens=max_tokens, act_dtype=act)
        del w
    return _dev[key]
