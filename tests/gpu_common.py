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
# The 2-bit codes enter the fp16 dot products as subnormals, whose products the
# instruction rounds on gfx950 (a probe: up to 3.1e-4 relative, typically far
# less), a second random error of the same order.  The check takes 4x the
# h-rounding figure.
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
    if kind == "ds4_ties_half":
        # router rows 4j+1 copy rows 4j: half the experts have an exact twin, so
        # the k-th / (k+1)-th boundary often falls between two equal logits
        # (whose experts have different weights)
        base = host_layer("ds4")
        lay = synth.Layer(**{**base.__dict__})
        r = base.router.copy()
        r[1::4] = r[0::4]
        lay.router = r
        return lay
    if kind == "tiny_hash":
        base = host_layer("tiny")
        lay = synth.Layer(**{**base.__dict__})
        lay.hash_table = synth.hash_table(0, 1000, base.spec.n_expert, base.spec.top_k)
        return lay
    if kind == "ds4_hash":
        # a hash layer of the model's shape: a table over the full vocabulary
        base = host_layer("ds4")
        lay = synth.Layer(**{**base.__dict__})
        lay.hash_table = synth.hash_table(1, synth.N_VOCAB, base.spec.n_expert, base.spec.top_k)
        return lay
    if kind == "tiny_noshared":
        return synth.make_layer(synth.TINY, seed=5, shared=False)
    if kind == "ds4_zipf":
        base = host_layer("ds4")
        lay = synth.Layer(**{**base.__dict__})
        lay.router_bias = synth.zipf_router_bias(1, 256)
        return lay
    raise KeyError(kind)


_dev = {}


def device_layer(kind: str, max_tokens: int = 64, act=None):
    """A MoELayer handle (cached per kind, max_tokens and activation dtype;
    by default fp32 activations for the tiny kinds, bf16 for the others)."""
    import bit_quantized_moe_renorm_amd as m
    if act is None:
        act = m.F32 if kind.startswith("tiny") else m.BF16
    key = (kind, max_tokens, act)
    if key not in _dev:
        lay = host_layer(kind)
        log(f"[gpu] create layer {kind} max_tokens={max_tokens} act={act}")
        w = m.upload_layer(lay)
        _dev[key] = m.MoELayer(lay.spec, w, max_tokens=max_tokens, act_dtype=act)
        del w
    return _dev[key]


def tie_split_tokens(kind: str, x_np, want: int):
    """Indices of tokens (up to ``want``) whose oracle top-k boundary falls
    between two experts with exactly equal fp32 logits: the k-th selected
    expert has a twin outside the selection, so only the lower-index rule
    decides which of the two is taken."""
    import oracle
    lay = host_layer(kind)
    lg, idx, _, _ = oracle.route(x_np, lay.router, lay.router_bias, lay.spec.top_k)
    out = []
    for t in range(len(x_np)):
        last = idx[t, -1]
        twins = np.nonzero(lg[t] == lg[t, last])[0]
        if any(e not in idx[t] for e in twins):
            out.append(t)
        if len(out) == want:
            break
    return np.array(out, dtype=np.int64)
