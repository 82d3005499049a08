"""Pins for the oracle's block output and RMSNorm (CPU only).

The block output is checked against a textbook dense SwiGLU mixture written
with numpy float64 matmuls on the (separately pinned) dequantised matrices,
and against invariants: zeroed experts, identical experts, top-1, token
permutation, no shared expert.
"""
import copy

import numpy as np
import pytest
from scipy.special import expit, softmax

from bit_quantized_moe_renorm_amd import synth


def _dense_reference(oracle, layer, x64, idx, w):
    """sum_j w_j * Wd (silu(Wg x) * (Wu x)) + shared, with numpy matmuls."""
    n, E = x64.shape
    out = np.zeros((n, E))
    for t in range(n):
        for j in range(idx.shape[1]):
            e = int(idx[t, j])
            Wg = oracle.dequant_matrix(layer, e, "gate").astype(np.float64)
            Wu = oracle.dequant_matrix(layer, e, "up").astype(np.float64)
            Wd = oracle.dequant_matrix(layer, e, "down").astype(np.float64)
            g, u = Wg @ x64[t], Wu @ x64[t]
            out[t] += w[t, j] * (Wd @ (g * expit(g) * u))
        if layer.sh_gate is not None:
            Sg = synth.bf16_bits_to_f32(layer.sh_gate).astype(np.float64)
            Su = synth.bf16_bits_to_f32(layer.sh_up).astype(np.float64)
            Sd = synth.bf16_bits_to_f32(layer.sh_down).astype(np.float64)
            g, u = Sg @ x64[t], Su @ x64[t]
            out[t] += Sd @ (g * expit(g) * u)
    return out


@pytest.fixture(scope="module")
def tiny():
    return synth.make_layer(synth.TINY, seed=0)


def test_tiny_matches_dense_swiglu(oracle_lib, tiny):
    x = synth.activations(0, 4, 256, bf16=False)
    out, idx, w = oracle_lib.forward(tiny, x)
    lg, idx2, _, w2 = oracle_lib.route(x, tiny.router, None, 2)
    assert np.array_equal(idx, idx2)
    # independent weights: softmax over the selected logits (scipy)
    wref = np.stack([softmax(lg[t][idx[t]].astype(np.float64)) for t in range(4)])
    ref = _dense_reference(oracle_lib, tiny, x.astype(np.float64), idx, wref)
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_ds4_shape_one_token_matches_dense(oracle_lib):
    """One DS4-shape token (6 of 256 experts + shared) against numpy matmuls."""
    spec = synth.LayerSpec(n_embd=4096, n_ff=2048, n_expert=16, top_k=6)
    layer = synth.make_layer(spec, seed=1)
    x = synth.activations(1, 1, 4096)
    out, idx, w = oracle_lib.forward(layer, x)
    x64 = synth.bf16_bits_to_f32(x).astype(np.float64)
    ref = _dense_reference(oracle_lib, layer, x64, idx, w)
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_zero_experts_leave_shared_only(oracle_lib, tiny):
    lay = copy.deepcopy(tiny)
    lay.gate[..., 0:2] = 0      # d = 0
    lay.up[..., 0:2] = 0
    lay.down[..., 80:84] = 0    # d = dmin = 0
    x = synth.activations(0, 4, 256, bf16=False)
    out, idx, w = oracle_lib.forward(lay, x)
    ref = _dense_reference(oracle_lib, lay, x.astype(np.float64), idx, np.zeros_like(w))
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))
    # and with no shared expert either, the block contributes exactly zero
    lay.sh_gate = lay.sh_up = lay.sh_down = None
    out0, _, _ = oracle_lib.forward(lay, x)
    assert np.all(out0 == 0)


def test_identical_experts_reduce_to_one(oracle_lib, tiny):
    """All experts equal: the weights sum to 1, so out = FFN_0(x) + shared."""
    lay = copy.deepcopy(tiny)
    for e in range(1, lay.spec.n_expert):
        lay.gate[e] = lay.gate[0]
        lay.up[e] = lay.up[0]
        lay.down[e] = lay.down[0]
    x = synth.activations(0, 4, 256, bf16=False)
    out, idx, w = oracle_lib.forward(lay, x)
    one = np.zeros_like(idx)
    ref = _dense_reference(oracle_lib, lay, x.astype(np.float64), one[:, :1], np.ones((4, 1)))
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_top1_uses_weight_one(oracle_lib):
    spec = synth.LayerSpec(n_embd=256, n_ff=256, n_expert=8, top_k=1)
    lay = synth.make_layer(spec, seed=3, shared=False)
    x = synth.activations(3, 3, 256)
    out, idx, w = oracle_lib.forward(lay, x)
    assert np.all(w == 1.0)
    x64 = synth.bf16_bits_to_f32(x).astype(np.float64)
    ref = _dense_reference(oracle_lib, lay, x64, idx, np.ones((3, 1)))
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_token_permutation_and_row_subset(oracle_lib, tiny):
    x = synth.activations(5, 6, 256, bf16=False)
    out, idx, _ = oracle_lib.forward(tiny, x)
    perm = np.array([3, 0, 5, 1, 4, 2])
    outp, idxp, _ = oracle_lib.forward(tiny, x[perm])
    assert np.array_equal(outp, out[perm]) and np.array_equal(idxp, idx[perm])
    rows = np.array([4, 1], np.int32)
    outr, _, _ = oracle_lib.forward(tiny, x, rows)
    assert np.array_equal(outr, out[rows])


def test_rmsnorm_pins(oracle_lib):
    # constant vector c -> c / sqrt(c^2 + eps)
    for c in (0.5, -3.0, 1e-4):
        h = np.full((1, 64), c, np.float32)
        _, x64 = oracle_lib.rmsnorm(h, 1e-6)
        assert np.allclose(x64, c / np.sqrt(c * c + 1e-6), rtol=1e-15)
    rng = np.random.default_rng(2)
    h = (rng.standard_normal((8, 4096)) * 3).astype(np.float32)
    xb, x64 = oracle_lib.rmsnorm(h, 1e-6)
    # unit RMS (eps negligible here) and scale invariance
    assert np.allclose(np.sqrt((x64 ** 2).mean(1)), 1.0, rtol=1e-6)
    # with eps = 0, scaling h by a power of two leaves x unchanged exactly
    _, x64a = oracle_lib.rmsnorm(h, 0.0)
    _, x64b = oracle_lib.rmsnorm(h * np.float32(4.0), 0.0)
    assert np.array_equal(x64b, x64a)
    # bf16 output is one of the two bf16 neighbours of the fp64 value, the nearer one
    xf = synth.bf16_bits_to_f32(xb).astype(np.float64)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(x64))) - 7)
    assert np.all(np.abs(xf - x64) <= ulp / 2 * (1 + 1e-12))


def test_forward_rejects_bad_shapes(oracle_lib):
    lib = oracle_lib.lib()
    rc = lib.oracle_forward(100, 256, 8, 2, 0, *([None] * 10), 0, None, 0, None, None, 0, None, None, None)
    assert rc == -1
    # an unknown expert format
    rc = lib.oracle_forward(256, 256, 8, 2, 2, *([None] * 10), 0, None, 0, None, None, 0, None, None, None)
    assert rc == -1


def test_stack_of_silent_layers_keeps_the_residual(oracle_lib, tiny):
    """Layers whose block contributes exactly zero (routed scales 0, no shared
    expert) leave the residual stream unchanged, and every layer sees the same
    normalised input."""
    lay = copy.deepcopy(tiny)
    lay.gate[..., 0:2] = 0
    lay.up[..., 0:2] = 0
    lay.down[..., 80:84] = 0
    lay.sh_gate = lay.sh_up = lay.sh_down = None
    h0 = synth.residual(3, 4, 256)
    h, xs, idxs, _ = oracle_lib.stack([lay, lay, lay], h0)
    assert np.array_equal(h, h0)
    x0, _ = oracle_lib.rmsnorm(h0, 1e-6)
    assert all(np.array_equal(x, x0) for x in xs)
    assert all(np.array_equal(i, idxs[0]) for i in idxs)


def test_stack_norm_before_block_and_residual_add(oracle_lib, tiny):
    """With eps = 0 the norm is exactly scale-invariant (a power-of-two scale),
    so the first layer's contribution does not change when h0 is doubled:
    h1(2 h0) - 2 h0 == h1(h0) - h0 up to the fp32 rounding of the stream.  A
    norm applied after the block, or a dropped residual, breaks this."""
    lay2 = synth.make_layer(synth.TINY, seed=5)
    h0 = synth.residual(4, 4, 256)
    a, _, _, _ = oracle_lib.stack([tiny], h0, eps=0.0)
    b, _, _, _ = oracle_lib.stack([tiny], 2 * h0, eps=0.0)
    da = a.astype(np.float64) - h0
    db = b.astype(np.float64) - 2 * h0.astype(np.float64)
    # each stream value is one fp32 rounding of an fp64 sum: half an ulp each
    ulp = np.spacing(np.maximum(np.abs(a), np.abs(b))).astype(np.float64)
    assert np.all(np.abs(da - db) <= ulp)
    assert np.max(np.abs(da)) > 1e-3          # the block does contribute
    # two layers: the second sees the first layer's updated stream
    _, xs, _, _ = oracle_lib.stack([tiny, lay2], h0)
    h1, _, _, _ = oracle_lib.stack([tiny], h0)
    x1, _ = oracle_lib.rmsnorm(h1, 1e-6)
    assert np.array_equal(xs[1], x1)
