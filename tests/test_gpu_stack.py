"""GPU parity of a stack of DS4-shape layers (RMSNorm, MoE block, residual add)
against the oracle's stack, both running free from the same seeded inputs.

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


@functools.lru_cache(maxsize=1)
def _case():
    layers = [synth.make_layer(synth.DS4, seed=SEED0 + l) for l in range(N_LAYERS)]
    h0 = synth.residual(40, N_TOK, 4096)
    return layers, h0, oracle.stack(layers, h0)


@pytest.mark.parametrize("per_token", [True, False], ids=["decode_b1", "batch4"])
def test_stack_matches_oracle(per_token):
    layers, h0, (ref_h, ref_x, ref_idx, ref_logits) = _case()

    devs = []
    for l, lay in enumerate(layers):
        log(f"[gpu] stack: create layer {l} (seed {SEED0 + l})")
        w = m.upload_layer(lay)
        devs.append(m.MoELayer(lay.spec, w, max_tokens=N_TOK))
        del w
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
    for dev in devs:
        dev.close()

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
    devs = []
    for l, lay in enumerate(layers):
        log(f"[gpu] forward_stack: create layer {l} (seed {SEED0 + l})")
        w = m.upload_layer(lay)
        devs.append(m.MoELayer(lay.spec, w, max_tokens=N_TOK))
        del w
    h = torch.from_numpy(h0.copy()).cuda()
    if per_token:
        for t in range(N_TOK):
            m.forward_stack(devs, h[t:t + 1])
    else:
        m.forward_stack(devs, h)
    torch.cuda.synchronize()
    got_h = h.cpu().numpy()
    for dev in devs:
        dev.close()
    err = rel_err(got_h.astype(np.float64) - h0, ref_h.astype(np.float64) - h0)
    log(f"[gpu] forward_stack of {N_LAYERS} ({'decode b=1' if per_token else 'batch of 4'}): "
        f"rel err of the accumulated block outputs {err:.3e}")
    assert err <= REL_TOL
    assert np.all(np.isfinite(got_h))
