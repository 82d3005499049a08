"""Pins for the oracle's hash-routed layers (CPU only).

The pages name the model's hash layers (the constant DS4_N_HASH_LAYER = 3 in
the model-constants listing of "DS4 ... 2.1 model architecture") and nothing
more.  The reading pinned here: a hash layer takes a token's k experts from a
fixed table indexed by the token's id, in the table's slot order, and weights
them by the router's softmax renormalised over those k experts.

Pins: where the table row is the token's own learned top-k the hashed route
reduces to the learned one (whose weights are pinned against scipy in the
routing pins); weight ratios equal exp of logit differences (scipy); the block
output equals a dense numpy SwiGLU mixture over the table's experts; ids out
of range are refused; the ids, not the activations, pick the experts.
"""
import numpy as np
import pytest
from scipy.special import softmax

from bit_quantized_moe_renorm_amd import synth
from test_oracle_forward import _dense_reference


@pytest.fixture(scope="module")
def tiny_hashed():
    lay = synth.make_layer(synth.TINY, seed=0)
    lay.hash_table = synth.hash_table(0, 64, lay.spec.n_expert, lay.spec.top_k)
    return lay


def test_table_shape_and_distinct_experts():
    tab = synth.hash_table(7, 1000, 256, 6)
    assert tab.shape == (1000, 6) and tab.dtype == np.int32
    assert tab.min() >= 0 and tab.max() < 256
    assert all(len(set(r)) == 6 for r in tab.tolist())
    # every expert is used (uniform draw over 6000 slots)
    assert len(np.unique(tab)) == 256
    assert np.array_equal(tab, synth.hash_table(7, 1000, 256, 6))


def test_reduces_to_learned_route(oracle_lib):
    """Table row = the token's learned top-k (in the learned slot order): the
    experts and weights equal the learned router's."""
    spec = synth.LayerSpec(n_embd=512, n_ff=256, n_expert=64, top_k=6)
    lay = synth.make_layer(spec, seed=2)
    x = synth.activations(2, 16, 512)
    _, idx, _, w64 = oracle_lib.route(x, lay.router, lay.router_bias, 6)
    ids = np.arange(16, dtype=np.int32)
    _, hidx, _, hw64 = oracle_lib.route_hashed(x, lay.router, lay.router_bias, 6, ids, idx)
    assert np.array_equal(hidx, idx)
    assert np.max(np.abs(hw64 - w64)) <= 4e-16


def test_weights_follow_softmax_of_table_logits(oracle_lib):
    spec = synth.LayerSpec(n_embd=512, n_ff=256, n_expert=64, top_k=6)
    lay = synth.make_layer(spec, seed=3)
    tab = synth.hash_table(3, 100, 64, 6)
    x = synth.activations(3, 12, 512)
    ids = synth.token_ids(3, 12, 100)
    lg, idx, w, w64 = oracle_lib.route_hashed(x, lay.router, lay.router_bias, 6, ids, tab)
    assert np.array_equal(idx, tab[ids])
    for t in range(12):
        ref = softmax(lg[t][tab[ids[t]]].astype(np.float64))
        assert np.max(np.abs(w64[t] - ref)) <= 1e-15
        assert abs(w64[t].sum() - 1.0) <= 1e-15 and np.all(w64[t] > 0)
    assert np.array_equal(w, w64.astype(np.float32))
    # the logits are the learned router's (hashing changes only the selection)
    lg2, _, _, _ = oracle_lib.route(x, lay.router, lay.router_bias, 6)
    assert np.array_equal(lg, lg2)


def test_forward_matches_dense_swiglu(oracle_lib, tiny_hashed):
    x = synth.activations(0, 5, 256, bf16=False)
    ids = synth.token_ids(0, 5, 64)
    out, idx, w = oracle_lib.forward(tiny_hashed, x, token_ids=ids)
    assert np.array_equal(idx, tiny_hashed.hash_table[ids])
    lg, _, _, _ = oracle_lib.route(x, tiny_hashed.router, None, 2)
    wref = np.stack([softmax(lg[t][idx[t]].astype(np.float64)) for t in range(5)])
    ref = _dense_reference(oracle_lib, tiny_hashed, x.astype(np.float64), idx, wref)
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_ids_pick_the_experts(oracle_lib, tiny_hashed):
    """One activation row under two ids: the experts are the two table rows."""
    x = np.repeat(synth.activations(1, 1, 256, bf16=False), 2, axis=0)
    tab = tiny_hashed.hash_table
    a, b = next((i, j) for i in range(64) for j in range(64) if set(tab[i]) != set(tab[j]))
    out, idx, _ = oracle_lib.forward(tiny_hashed, x, token_ids=np.array([a, b], np.int32))
    assert np.array_equal(idx, tab[[a, b]])
    assert not np.array_equal(out[0], out[1])
    # rows and ids permute together
    out2, idx2, _ = oracle_lib.forward(tiny_hashed, x[::-1].copy(), token_ids=np.array([b, a], np.int32))
    assert np.array_equal(out2, out[::-1]) and np.array_equal(idx2, idx[::-1])


def test_out_of_range_ids_are_refused(oracle_lib, tiny_hashed):
    x = synth.activations(0, 2, 256, bf16=False)
    with pytest.raises(AssertionError):
        oracle_lib.route_hashed(x, tiny_hashed.router, None, 2, np.array([0, 64], np.int32),
                                tiny_hashed.hash_table)
    with pytest.raises(AssertionError):
        oracle_lib.forward(tiny_hashed, x, token_ids=np.array([-1, 3], np.int32))


def test_stack_routes_hash_layers_by_id(oracle_lib, tiny_hashed):
    lay2 = synth.make_layer(synth.TINY, seed=5)
    h0 = synth.residual(4, 6, 256)
    ids = synth.token_ids(4, 6, 64)
    h, xs, idxs, _ = oracle_lib.stack([tiny_hashed, lay2], h0, token_ids=ids)
    assert np.array_equal(idxs[0], tiny_hashed.hash_table[ids])
    _, ridx, _, _ = oracle_lib.route(xs[1], lay2.router, lay2.router_bias, 2)
    assert np.array_equal(idxs[1], ridx)
    # same as running the layers one at a time
    y0, _, _ = oracle_lib.forward(tiny_hashed, xs[0], token_ids=ids)
    h1 = (h0.astype(np.float64) + y0).astype(np.float32)
    x1, _ = oracle_lib.rmsnorm(h1, 1e-6)
    assert np.array_equal(x1, xs[1])
