"""GPU parity of a stack of DS4-shape layers (RMSNorm, MoE block, residual add).

Teacher-forced checks (the first two tests): each layer's GPU input x_l (the
bf16 RMSNorm of the GPU's own residual stream) is handed to the oracle, which
computes that layer's routing and block output from it; the GPU's routing must
match bit for bit and its block output within the bar, layer by layer.  This
is the per-layer contract; errors do not compound.

Free-running checks (the last two): both sides run the whole stack from the
same seeded h0.

Nothing is handed from one side to the other: each side normalises its own
residual stream.  The two streams agree to the block's own roundings per layer, so
the normalised inputs agree bit for bit except where a value sits at a bf16
rounding boundary.  The routing is compared wherever the x differences cannot
change it: each logit moves by at most |router row| . |x_gpu - x_ref|, so the
selected set (and its order) is checked for every token whose logit gaps exceed
those bounds.
"""
import functools

import numpy as np
import pytest

import oracle
from bit_quantized_moe_renorm_amd import synth
from gpu_common import REL_TOL, log, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_moe_renorm_amd as m  # noqa: E402

N_LAYERS, N_TOK = 3, 4
SEED0 = 4000  # layer l uses seed 4000 + l
CHUNK = 512


@functools.lru_cache(maxsize=1)
def _host_layers():
    return [synth.make_layer(synth.DS4, seed=SEED0 + l) for l in range(N_LAYERS)]


_DEVS = {}


def _device_layers():
    if not _DEVS:
        for l, lay in enumerate(_host_layers()):
            log(f"[gpu] stack: create layer {l} (seed {SEED0 + l}), max_tokens {CHUNK}")
            w = m.upload_layer(lay)
            _DEVS[l] = m.MoELayer(lay.spec, w, max_tokens=CHUNK)
            del w
    return [_DEVS[l] for l in range(N_LAYERS)]


def _teacher_forced(h0, per_token):
    """Run the stack layer by layer on the GPU, keeping each layer's input
    x_l, block output y_l (forward into zeros) and routing."""
    devs = _device_layers()
    n = h0.shape[0]
    h = torch.from_numpy(h0.copy()).cuda()
    rec = []
    for l, dev in enumerate(devs):
        hl = h.cpu().numpy()
        x = m.rmsnorm(h)
        y = torch.zeros_like(h)
        if per_token:
            idx = []
            for t in range(n):
                dev.forward(x[t:t + 1], y[t:t + 1])
                idx.append(dev.last_routing(1)[0])
            idx = torch.cat(idx)
        else:
            dev.forward(x, y)
            idx = dev.last_routing(n)[0]
        torch.cuda.synchronize()
        rec.append((hl, x.view(torch.int16).cpu().numpy().view(np.uint16), y.cpu().numpy(), idx.cpu().numpy()))
        h = h + y
    return rec


@pytest.mark.parametrize("per_token,n,sample", [(False, CHUNK, 32), (True, N_TOK, N_TOK)],
                         ids=["chunk512", "decode_b1"])
def test_stack_teacher_forced(per_token, n, sample):
    """Per layer: RMSNorm bit-exact against the oracle's on the GPU's own
    residual; routing of every token bit-exact; block output within the bar
    on a seeded sample of tokens (all of them for decode)."""
    layers = _host_layers()
    h0 = synth.residual(43, n, 4096)
    rec = _teacher_forced(h0, per_token)
    rows = np.sort(np.random.default_rng(5).choice(n, sample, replace=False)).astype(np.int32)
    for l, (hl, xl, yl, idx) in enumerate(rec):
        ref_x, _ = oracle.rmsnorm(hl, 1e-6)
        assert np.array_equal(xl, ref_x), f"layer {l}: RMSNorm differs"
        _, ridx, _, _ = oracle.route(xl, layers[l].router, layers[l].router_bias, layers[l].spec.top_k)
        assert np.array_equal(idx, ridx), f"layer {l}: routing differs"
        ref_y, _, _ = oracle.forward(layers[l], xl, rows=rows)
        err = rel_err(yl[rows], ref_y)
        log(f"[gpu] teacher-forced layer {l} ({'decode b=1' if per_token else f'{n}-token chunk'}): "
            f"routing of {n} tokens equal, block output rel err {err:.3e} on {len(rows)} tokens")
        assert err <= REL_TOL


def test_forward_stack_matches_layer_by_layer():
    """The one-call stack (RMSNorm + forward per layer in ds4moe_forward_stack)
    against the layer-by-layer run above, on a 512-token chunk.  One layer:
    the same input, so the whole chunk must agree within the bar.  Three
    layers: the two runs add the same contributions in a different order, and
    a last-bit difference in the residual can move an x_l value across a bf16
    rounding boundary and flip a near-tied routing downstream; every token
    but such rare ones must agree within the bar."""
    h0 = synth.residual(44, CHUNK, 4096)
    rec = _teacher_forced(h0, False)
    devs = _device_layers()
    h1 = torch.from_numpy(h0.copy()).cuda()
    m.forward_stack(devs[:1], h1)
    torch.cuda.synchronize()
    err1 = rel_err(h1.cpu().numpy().astype(np.float64) - h0, rec[0][2])
    log(f"[gpu] forward_stack vs layer by layer, 1 layer, 512 tokens: rel diff {err1:.3e}")
    assert err1 <= REL_TOL
    h_ref = rec[-1][0].astype(np.float64) + rec[-1][2] - h0
    h = torch.from_numpy(h0.copy()).cuda()
    m.forward_stack(devs, h)
    torch.cuda.synchronize()
    got = h.cpu().numpy().astype(np.float64) - h0
    per_tok = np.max(np.abs(got - h_ref), axis=1) / np.max(np.abs(h_ref))
    bad = int(np.count_nonzero(per_tok > REL_TOL))
    log(f"[gpu] forward_stack vs layer by layer, {N_LAYERS} layers, 512 tokens: {bad} tokens beyond the bar, "
        f"median rel diff {np.median(per_tok):.3e}")
    assert bad <= 5


@functools.lru_cache(maxsize=1)
def _case():
    layers = _host_layers()
    h0 = synth.residual(40, N_TOK, 4096)
    return layers, h0, oracle.stack(layers, h0)


@pytest.mark.parametrize("per_token", [True, False], ids=["decode_b1", "batch4"])
def test_stack_matches_oracle(per_token):
    layers, h0, (ref_h, ref_x, ref_idx, ref_logits) = _case()

    devs = _device_layers()
    h = torch.from_numpy(h0.copy()).cuda()
    xs, idxs = [], []
    for l, dev in enumerate(devs):
        x = m.rmsnorm(h)
        idx, _, _, _ = dev.route(x)
        if per_token:
            for t in range(N_TOK):
                dev.forward(x[t:t + 1], h[t:t + 1])
        else:
            dev.forward(x, h)
        xs.append(x.view(torch.int16).cpu().numpy().view(np.uint16))
        idxs.append(idx.cpu().numpy())
    torch.cuda.synchronize()
    got_h = h.cpu().numpy()

    k = layers[0].spec.top_k
    for l in range(N_LAYERS):
        nx = int(np.count_nonzero(xs[l] != ref_x[l]))
        # Each logit can move by at most |router row| . |x_gpu - x_ref| (plus a
        # few fp32 roundings): a comparison between two logits is decided where
        # their gap exceeds the sum of both bounds.
        xg = (xs[l].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        xr = (ref_x[l].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        lg = ref_logits[l].astype(np.float64)
        bound = np.abs(xg - xr) @ np.abs(layers[l].router.astype(np.float64)).T
        bound += 1e-6 * np.max(np.abs(lg), axis=1, keepdims=True)
        sel = ref_idx[l]
        lo_in = np.min(np.take_along_axis(lg - bound, sel, 1), axis=1)
        out_mask = np.ones_like(lg, dtype=bool)
        np.put_along_axis(out_mask, sel, False, 1)
        hi_out = np.max(np.where(out_mask, lg + bound, -np.inf), axis=1)
        set_decided = lo_in > hi_out
        lsel, bsel = np.take_along_axis(lg, sel, 1), np.take_along_axis(bound, sel, 1)
        order_decided = np.all(lsel[:, :-1] - bsel[:, :-1] > lsel[:, 1:] + bsel[:, 1:], axis=1)
        same_set = np.all(np.sort(idxs[l], 1) == np.sort(sel, 1), axis=1)
        same_order = np.all(idxs[l] == sel, axis=1)
        log(f"[gpu] stack layer {l}: x bits differing {nx}/{xs[l].size}, routing equal "
            f"{int(same_order.sum())}/{N_TOK} (sets {int(same_set.sum())}), decided sets "
            f"{int(set_decided.sum())}, decided orders {int(order_decided.sum())}")
        assert np.all(same_set[set_decided]), (l, idxs[l], sel)
        assert np.all(same_order[set_decided & order_decided]), (l, idxs[l], sel)
    contrib_gpu = got_h.astype(np.float64) - h0
    contrib_ref = ref_h.astype(np.float64) - h0
    err = rel_err(contrib_gpu, contrib_ref)
    log(f"[gpu] stack of {N_LAYERS} ({'decode b=1' if per_token else 'batch of 4'}): "
        f"rel err of the accumulated block outputs {err:.3e}")
    assert err <= REL_TOL
    assert np.all(np.isfinite(got_h))


@pytest.mark.parametrize("per_token", [True, False], ids=["decode_b1", "batch4"])
def test_forward_stack_matches_oracle(per_token):
    """The whole stack from one library call per token (or per batch)."""
    layers, h0, (ref_h, _, _, _) = _case()
    devs = _device_layers()
    h = torch.from_numpy(h0.copy()).cuda()
    if per_token:
        for t in range(N_TOK):
            m.forward_stack(devs, h[t:t + 1])
    else:
        m.forward_stack(devs, h)
    torch.cuda.synchronize()
    got_h = h.cpu().numpy()
    err = rel_err(got_h.astype(np.float64) - h0, ref_h.astype(np.float64) - h0)
    log(f"[gpu] forward_stack of {N_LAYERS} ({'decode b=1' if per_token else 'batch of 4'}): "
        f"rel err of the accumulated block outputs {err:.3e}")
    assert err <= REL_TOL
    assert np.all(np.isfinite(got_h))
