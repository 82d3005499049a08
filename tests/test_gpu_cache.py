"""Host-resident routed experts with an HBM expert cache, against the oracle.

The cache is a place for the weights, not a change of arithmetic: every
output must match the oracle (and the layer with all experts in HBM) on the
same inputs.  The cache policy (the call's resident experts are stamped, each
missing expert, in ascending order, takes a slot the call does not use:
empty ones first, then the least recently used, lower slot first on equal
stamps) is checked against a small model of that rule replayed on the
routing the library exported for each call.
"""
import numpy as np
import pytest

import oracle
from bit_quantized_moe_renorm_amd import synth
from gpu_common import FUSED_TOL, GEMV_TOL, REL_TOL, host_layer, log, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_moe_renorm_amd as m  # noqa: E402


class LruModel:
    """The cache rule, written out for the test."""

    def __init__(self, slots):
        self.expert = [-1] * slots
        self.stamp = [0] * slots
        self.clock = 0
        self.hits = self.misses = 0

    def call(self, experts):
        self.clock += 1
        now = self.clock
        where = {e: s for s, e in enumerate(self.expert) if e >= 0}
        missing = []
        for e in sorted(set(int(v) for v in experts)):
            if e in where:
                self.stamp[where[e]] = now
                self.hits += 1
            else:
                missing.append(e)
        free = sorted((st, s) for s, st in enumerate(self.stamp) if st != now)
        for e, (_, s) in zip(missing, free):
            self.expert[s] = e
            self.stamp[s] = now
            self.misses += 1


_cache_dev = {}


def cache_layer(kind, slots, max_tokens=64):
    key = (kind, slots, max_tokens)
    if key not in _cache_dev:
        lay = host_layer(kind)
        log(f"[gpu] create {kind} with {slots} cache slots")
        act = m.F32 if kind.startswith("tiny") else m.BF16
        _cache_dev[key] = m.MoELayer(lay.spec, m.upload_layer(lay), max_tokens=max_tokens, act_dtype=act,
                                     cache_slots=slots)
    return _cache_dev[key]


def _fwd(dev, x_np, ids=None):
    x = m.to_device_x(x_np)
    out = torch.zeros((x.shape[0], dev.spec.n_embd), dtype=torch.float32, device="cuda")
    dev.forward(x, out, ids=None if ids is None else m.to_device_ids(ids))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_decode_stream_matches_oracle_and_lru_model():
    """16 slots, 24 decode tokens one at a time (the fused decode kernel, fed
    the router kernel's routing after the cache step): every output against
    the oracle, every call's hits and misses and the final slot contents
    against the model of the rule."""
    lay = host_layer("ds4")
    dev = m.MoELayer(lay.spec, m.upload_layer(lay), max_tokens=8, act_dtype=m.BF16, cache_slots=16)
    x = synth.activations(11, 24, 4096)
    # repeats: tokens 12..17 are tokens 0..5 again (their experts may still be resident)
    x[12:18] = x[0:6]
    ref, ridx, _ = oracle.forward(lay, x)
    model = LruModel(16)
    for t in range(24):
        got = _fwd(dev, x[t:t + 1])
        err = rel_err(got, ref[t:t + 1])
        idx = dev.last_routing(1)[0].cpu().numpy()[0]
        assert np.array_equal(idx, ridx[t])
        model.call(idx)
        st = dev.cache_stats()
        log(f"[gpu] cache decode token {t}: rel err {err:.2e}, hits {st['hits']} misses {st['misses']}")
        assert err <= FUSED_TOL
        assert (st["calls"], st["hits"], st["misses"]) == (t + 1, model.hits, model.misses)
        assert st["bytes"] == model.misses * synth.layer_nbytes(lay.spec)["per_expert"]
    assert dev.cache_slots_held() == model.expert
    assert model.hits > 0                       # the repeated tokens found experts resident
    dev.close()


def test_cache_matches_resident_layer_gemv():
    """The same 3 tokens on the GEMV path through a 6-slot cache and with every
    expert in HBM: the same kernels, so the same values up to the atomics'
    order."""
    lay = host_layer("ds4")
    x = synth.activations(12, 3, 4096)
    a = cache_layer("ds4", 6)
    a.set_path(m.PATH_GEMV)
    got = _fwd(a, x)                            # 3 sub-calls of one token (6 slots / top-6)
    a.set_path(m.PATH_AUTO)
    b = m.MoELayer(lay.spec, m.upload_layer(lay), max_tokens=8, act_dtype=m.BF16)
    b.set_path(m.PATH_GEMV)
    want = _fwd(b, x)
    b.close()
    assert rel_err(got, want) <= 1e-6


@pytest.mark.parametrize("slots,n", [(64, 40), (256, 300)])
def test_batched_calls_through_the_cache(slots, n):
    """64 slots: a 40-token call runs as sub-calls of 10 tokens (grouped GEMMs);
    256 slots: one call holds every expert.  A second identical call misses
    nothing new once every expert it needs fits."""
    lay = host_layer("ds4")
    dev = cache_layer("ds4", slots, max_tokens=512)
    x = synth.activations(13, n, 4096)
    got = _fwd(dev, x)
    rows = np.unique(np.concatenate([[0, 1, 9, 10, n - 1], np.random.default_rng(n).choice(n, 20, replace=False)]))
    ref, _, _ = oracle.forward(lay, x, rows.astype(np.int32))
    err = rel_err(got[rows], ref)
    st = dev.cache_stats()
    log(f"[gpu] cache {slots} slots, {n} tokens: rel err {err:.2e}, stats {st}")
    assert err <= REL_TOL
    if slots == 256:
        _fwd(dev, x)
        st2 = dev.cache_stats()
        assert st2["misses"] == st["misses"] and st2["calls"] == st["calls"] + 1


def test_dequantize_reads_the_host_store():
    lay = host_layer("ds4")
    dev = cache_layer("ds4", 6)
    for e in (0, 131, 255):
        for which, name in enumerate(("gate", "up", "down")):
            got = dev.dequantize(e, which).cpu().numpy()
            assert np.array_equal(got.view(np.uint32), oracle.dequant_matrix(lay, e, name).view(np.uint32))


def test_q4_and_hash_layers_through_the_cache():
    base = synth.make_layer(synth.DS4, seed=1, fmt="q4")
    x = synth.activations(14, 5, 4096)
    log("[gpu] create q4 layer with 12 cache slots")
    dev = m.MoELayer(base.spec, m.upload_layer(base), max_tokens=8, act_dtype=m.BF16, cache_slots=12)
    got = _fwd(dev, x)                          # sub-calls of 2 tokens
    ref, _, _ = oracle.forward(base, x)
    assert rel_err(got, ref) <= REL_TOL
    assert dev.cache_stats()["calls"] == 3
    dev.close()
    lay = host_layer("ds4_hash")
    ids = synth.token_ids(14, 5, synth.N_VOCAB)
    dev = cache_layer("ds4_hash", 16)
    got = _fwd(dev, x, ids)
    ref, _, _ = oracle.forward(lay, x, token_ids=ids)
    assert rel_err(got, ref) <= REL_TOL


def test_tiny_fp32_cache():
    lay = host_layer("tiny")
    dev = cache_layer("tiny", 2)                # top-2: one token per sub-call
    x = synth.activations(15, 6, 256, bf16=False)
    got = _fwd(dev, x)                          # the fused kernel, one token at a time
    ref, _, _ = oracle.forward(lay, x)
    assert rel_err(got, ref) <= FUSED_TOL
    assert dev.cache_stats()["calls"] == 6


def test_cache_errors():
    dev = cache_layer("ds4", 6)
    x = m.to_device_x(synth.activations(1, 1, 4096))
    out = torch.zeros((1, 4096), dtype=torch.float32, device="cuda")
    with pytest.raises(m.Ds4MoeError) as ei:
        dev.forward_static(x, out)
    assert ei.value.code == m.EUNSUPPORTED
    lay = host_layer("tiny")
    plain = m.MoELayer(lay.spec, m.upload_layer(lay), max_tokens=4, act_dtype=m.F32)
    with pytest.raises(m.Ds4MoeError) as ei:
        plain.cache_stats()
    assert ei.value.code == m.EUNSUPPORTED
    plain.close()
