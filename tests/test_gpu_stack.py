"""GPU parity of a stack of DS4-shape layers (RMSNorm, MoE block, residual add)
against the oracle's stack, both running free from the same seeded inputs.

Nothing is handed from one side to the other: each side normalises its own
residual stream.  The two streams agree to a few fp32 roundings per layer, so
the normalised inputs agree bit for bit except where a value sits at a bf16
rounding boundary; the routing is compared wherever the oracle's own margin
between the k-th and (k+1)-th logit is wide enough to rule out such a flip.
"""
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


def _layers():
    return [synth.make_layer(synth.DS4, seed=SEED0 + l) for l in range(N_LAYERS)]


@pytest.mark.parametrize("per_token", [True, False], ids=["decode_b1", "batch4"])
def test_stack_matches_oracle(per_token):
    layers = _layers()
    h0 = synth.residual(40, N_TOK, 4096)
    ref_h, ref_x, ref_idx, ref_logits = oracle.stack(layers, h0)

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
        lg = np.sort(ref_logits[l], axis=1)[:, ::-1]
        margin = (lg[:, k - 1] - lg[:, k]) / np.maximum(np.abs(lg[:, k - 1]), 1e-30)
        wide = margin > 1e-4
        same = np.all(idxs[l] == ref_idx[l], axis=1)
        log(f"[gpu] stack layer {l}: x bits differing {nx}/{xs[l].size}, routing equal "
            f"{int(same.sum())}/{N_TOK}, oracle margins {np.round(margin, 6).tolist()}")
        assert np.all(same[wide]), (l, idxs[l], ref_idx[l])
    contrib_gpu = got_h.astype(np.float64) - h0
    contrib_ref = ref_h.astype(np.float64) - h0
    err = rel_err(contrib_gpu, contrib_ref)
    log(f"[gpu] stack of {N_LAYERS} ({'decode b=1' if per_token else 'batch of 4'}): "
        f"rel err of the accumulated block outputs {err:.3e}")
    assert err <= REL_TOL
    assert np.all(np.isfinite(got_h))
