"""Pins for the oracle's router and bucketing (CPU only).

Logits are pinned by inputs with exactly known dot products; top-k by brute
force over all k-subsets; the renormalised weights by scipy's softmax over the
selected logits (the oracle instead divides softmax probabilities by their
selected sum); the buckets by a brute-force filter.
"""
import itertools

import numpy as np
import pytest
from scipy.special import softmax

from bit_quantized_moe_renorm_amd import synth


def _route_logits(oracle, logits, k, bias=None):
    """Drive the router so that its logits equal `logits` exactly: x = e_0, R[:, 0] = logits."""
    n, ne = logits.shape
    E = 4
    x = np.zeros((n, E), np.float32)
    x[:, 0] = 1.0
    outs = []
    for t in range(n):
        R = np.zeros((ne, E), np.float32)
        R[:, 0] = logits[t]
        lg, idx, w, w64 = oracle.route(x[t:t + 1], R, bias, k)
        outs.append((lg[0], idx[0], w[0], w64[0]))
    return outs


def test_logits_exact_closed_form(oracle_lib):
    rng = np.random.default_rng(0)
    # integer-valued router and activations: the dot products are exact integers
    R = rng.integers(-50, 50, (16, 256)).astype(np.float32)
    x = rng.integers(-3, 4, (5, 256)).astype(np.float32)
    lg, _, _, _ = oracle_lib.route(x, R, None, 2)
    assert np.array_equal(lg, (x.astype(np.int64) @ R.T.astype(np.int64)).astype(np.float32))
    # one-hot activations pick a router column; bias is added
    xb = np.zeros((1, 256), np.float32)
    xb[0, 17] = 1.0
    bias = rng.standard_normal(16).astype(np.float32)
    lg, _, _, _ = oracle_lib.route(xb, R, bias, 2)
    assert np.array_equal(lg[0], (R[:, 17].astype(np.float64) + bias).astype(np.float32))
    # bf16 activations are read as bf16 bit patterns
    xbf = synth.f32_to_bf16_bits(x)
    lg2, _, _, _ = oracle_lib.route(xbf, R, None, 2)
    assert np.array_equal(lg2, (x.astype(np.int64) @ R.T.astype(np.int64)).astype(np.float32))


def test_logits_fp64_accumulation(oracle_lib):
    """A sum whose fp32 accumulation would lose the small terms is exact in the oracle."""
    E = 256
    R = np.zeros((2, E), np.float32)
    R[0, 0] = 2.0 ** 24
    R[0, 1:] = 1.0
    R[1, :] = 1.0
    x = np.ones((1, E), np.float32)
    lg, _, _, _ = oracle_lib.route(x, R, None, 1)
    assert lg[0, 0] == np.float32(2.0 ** 24 + 255)
    assert lg[0, 1] == 256.0


@pytest.mark.parametrize("ne,k", [(8, 2), (6, 3), (10, 4), (12, 6), (7, 1)])
def test_topk_brute_force(oracle_lib, ne, k):
    rng = np.random.default_rng(ne * 31 + k)
    logits = rng.standard_normal((6, ne)).astype(np.float32) * 2
    # inject exact ties at the k-th place in some rows
    logits[1, :] = np.round(logits[1, :])
    logits[2, :] = 0.5
    for t, (lg, idx, w, w64) in enumerate(_route_logits(oracle_lib, logits, k)):
        p = softmax(logits[t].astype(np.float64))
        # brute force: the k-subset with the largest probability mass; among equal
        # masses the lexicographically smallest index set (lower index wins ties)
        best = None
        for sub in itertools.combinations(range(ne), k):
            key = (np.float64(sum(sorted(logits[t][list(sub)].astype(np.float64)))), [-i for i in sub])
            if best is None or key > best[0]:
                best = (key, sub)
        assert sorted(idx.tolist()) == sorted(best[1]), (t, idx, best)
        # slots in decreasing logit, ascending index among equals
        order = sorted(range(ne), key=lambda e: (-logits[t][e], e))[:k]
        assert idx.tolist() == order
        # renormalised weights = softmax restricted to the selected experts
        ref = softmax(logits[t][idx].astype(np.float64))
        assert np.allclose(w64, ref, rtol=1e-14, atol=0)
        assert abs(w64.sum() - 1.0) < 1e-14
        assert np.array_equal(w, w64.astype(np.float32))
        # and it is NOT the unrenormalised softmax (unless k == ne)
        assert not np.allclose(w64, p[idx]) or k == ne


def test_all_equal_logits(oracle_lib):
    logits = np.zeros((1, 8), np.float32)
    lg, idx, w, w64 = _route_logits(oracle_lib, logits, 3)[0]
    assert idx.tolist() == [0, 1, 2]
    assert np.allclose(w64, 1 / 3, rtol=0, atol=1e-16)


def test_tie_at_kth_place_lower_index_wins(oracle_lib):
    logits = np.array([[0.0, 3.0, 1.0, 2.0, 1.0, 1.0]], np.float32)
    _, idx, _, _ = _route_logits(oracle_lib, logits, 3)[0]
    assert idx.tolist() == [1, 3, 2]


def test_k1_weight_is_one(oracle_lib):
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((4, 9)).astype(np.float32)
    for lg, idx, w, w64 in _route_logits(oracle_lib, logits, 1):
        assert w64[0] == 1.0


def test_shift_and_unselected_invariance(oracle_lib):
    """Weights do not change when all logits shift by a constant (exact here: integer
    logits) or when unselected logits move while staying below the k-th."""
    rng = np.random.default_rng(6)
    base = rng.integers(-8, 8, (1, 12)).astype(np.float32)
    _, idx, _, w0 = _route_logits(oracle_lib, base, 4)[0]
    _, idx1, _, w1 = _route_logits(oracle_lib, base + 5.0, 4)[0]
    assert idx.tolist() == idx1.tolist()
    assert np.allclose(w0, w1, rtol=1e-15, atol=0)
    kth = np.sort(base[0])[::-1][3]
    moved = base.copy()
    for e in range(12):
        if e not in idx:
            moved[0, e] = kth - 3.0 - e
    _, idx2, _, w2 = _route_logits(oracle_lib, moved, 4)[0]
    assert idx.tolist() == idx2.tolist()
    assert np.allclose(w0, w2, rtol=1e-15, atol=0)


def test_bias_changes_selection(oracle_lib):
    logits = np.zeros((1, 8), np.float32)
    bias = np.array([0, 0, 0, 0, 0, 0, 0, 1], np.float32)
    _, idx, _, _ = _route_logits(oracle_lib, logits, 2, bias=bias)[0]
    assert idx.tolist() == [7, 0]


def test_bucket_brute_force(oracle_lib):
    rng = np.random.default_rng(21)
    for n, k, ne in [(1, 6, 256), (4, 2, 8), (33, 6, 256), (200, 3, 16), (0, 2, 8)]:
        idx = np.array([rng.choice(ne, k, replace=False) for _ in range(n)], np.int32).reshape(n, k)
        off, tok = oracle_lib.bucket(idx, ne)
        assert off[0] == 0 and off[-1] == n * k
        assert np.all(np.diff(off) >= 0)
        for e in range(ne):
            expect = [t for t in range(n) if e in idx[t]]
            assert tok[off[e]:off[e + 1]].tolist() == expect
        # every token appears in exactly k lists
        assert np.array_equal(np.bincount(tok, minlength=n), np.full(n, k)) if n else True


def test_route_real_layer_consistency(oracle_lib):
    """On a DS4-shape router: Σw = 1, indices distinct, weights descending."""
    lay_router = (synth.rng_for(1, "router").standard_normal((256, 4096)) * 0.02).astype(np.float32)
    x = synth.activations(1, 16, 4096)
    lg, idx, w, w64 = oracle_lib.route(x, lay_router, None, 6)
    assert np.allclose(w64.sum(1), 1.0, rtol=0, atol=1e-14)
    for t in range(16):
        assert len(set(idx[t].tolist())) == 6
        assert np.all(np.diff(w64[t]) <= 0)
        assert np.all(lg[t][idx[t]] >= np.delete(lg[t], idx[t]).max())
