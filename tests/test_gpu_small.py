"""GPU parity of the small-batch kernels (2..8 bf16 tokens: the router, then
the two persistent MFMA launches) against the CPU oracle, through the C ABI.

These are the batch sizes of speculative (MTP) verification, which scores the
last token plus k drafted ones in one call ("ds4 深度实战...", sections 4.2 and
4.4), and of small-batch decode.  The kernels round the routed weights to fp16
as the grouped GEMMs do, and x and h to fp16 under power-of-two scales, with
fp32 accumulation: the bar is the batched paths' max|gpu - ref| / max|ref| <=
2e-3.  Each test also logs the measured error.
"""
import numpy as np
import pytest

import oracle
from bit_quantized_moe_renorm_amd import synth
from gpu_common import REL_TOL, device_layer, host_layer, log, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_moe_renorm_amd as m  # noqa: E402


def _forward(dev, x_np, path=None, out0=None, ids=None):
    """out0 + MoE(x) on the GPU; also returns the timing kinds the call used."""
    x = m.to_device_x(x_np)
    n = x.shape[0]
    out = torch.zeros((n, x.shape[1]), dtype=torch.float32, device="cuda")
    if out0 is not None:
        out.copy_(torch.from_numpy(out0))
    if path is not None:
        dev.set_path(path)
    dev.timing_enable(True)
    try:
        dev.forward(x, out, ids=None if ids is None else m.to_device_ids(ids))
        torch.cuda.synchronize()
        kinds = dev.timing_read()
    finally:
        dev.timing_enable(False)
        if path is not None:
            dev.set_path(m.PATH_AUTO)
    return out.cpu().numpy(), kinds


def _check(kind, lay, got, x, kinds, tag, ids=None):
    assert "small_gateup" in kinds and "small_down" in kinds, kinds
    ref, _, _ = oracle.forward(lay, x, token_ids=ids)
    err = rel_err(got, ref)
    log(f"[gpu] small {tag} rel err {err:.3e}")
    assert err <= REL_TOL


@pytest.mark.parametrize("kind", ["ds4", "ds4_zipf"])
@pytest.mark.parametrize("n", [2, 3, 5, 7, 8])
def test_small_matches_oracle(kind, n):
    """AUTO takes the small-batch kernels for 2..8 bf16 tokens; uniform and
    Zipf-skewed routing (many tokens per expert)."""
    lay = host_layer(kind)
    x = synth.activations(20 + n, n, lay.spec.n_embd)
    got, kinds = _forward(device_layer(kind), x)
    _check(kind, lay, got, x, kinds, f"{kind} n={n}")


def test_small_every_token_on_the_same_experts():
    """Eight copies of one token: every selected expert holds all 8 tokens
    (the largest token count a unit takes)."""
    lay = host_layer("ds4")
    x = np.repeat(synth.activations(40, 1, 4096), 8, axis=0)
    got, kinds = _forward(device_layer("ds4"), x, m.PATH_SMALL)
    _, idx, _, _ = oracle.route(x, lay.router, lay.router_bias, lay.spec.top_k)
    assert len(np.unique(idx)) == lay.spec.top_k
    _check("ds4", lay, got, x, kinds, "8 equal tokens")


@pytest.mark.parametrize("kind", ["tiny", "tiny_noshared"])
@pytest.mark.parametrize("n", [2, 4, 8])
def test_small_tiny_shapes(kind, n):
    """n_embd = n_ff = 256 (one 256-K block per row: units of one block), 8
    experts, top-2, with and without the shared expert, bf16 activations."""
    lay = host_layer(kind)
    x = synth.activations(50 + n, n, 256)
    got, kinds = _forward(device_layer(kind, 16, act=m.BF16), x)
    _check(kind, lay, got, x, kinds, f"{kind} n={n}")


def test_small_accumulates_into_residual():
    lay = host_layer("ds4")
    x = synth.activations(60, 5, 4096)
    out0 = synth.activations(61, 5, 4096, bf16=False)
    got, kinds = _forward(device_layer("ds4"), x, out0=out0)
    ref, _, _ = oracle.forward(lay, x)
    err = rel_err(got - out0, ref)
    log(f"[gpu] small residual rel err {err:.3e}")
    assert err <= REL_TOL


def test_small_calls_in_a_row_and_between_other_paths():
    """The two gate/up sum buffers alternate and each call clears the other:
    calls of varying size in a row, and with decode and GEMM calls between
    them, each against the oracle."""
    lay = host_layer("ds4_zipf")
    dev = device_layer("ds4_zipf")
    seq = [(8, None), (2, None), (5, None), (1, None), (8, None), (16, None), (3, None), (7, m.PATH_SMALL),
           (6, None)]
    for i, (n, path) in enumerate(seq):
        x = synth.activations(70 + i, n, 4096)
        got, kinds = _forward(dev, x, path)
        ref, _, _ = oracle.forward(lay, x)
        err = rel_err(got, ref)
        used = sorted(kinds)
        log(f"[gpu] call {i} n={n} kinds {used} rel err {err:.3e}")
        assert ("small_gateup" in kinds) == (2 <= n <= 8)
        assert err <= REL_TOL


def test_small_hash_layer():
    """A hash-routed layer's batch (experts from the table row of each token id)."""
    lay = host_layer("ds4_hash")
    n = 7
    x = synth.activations(80, n, 4096)
    ids = synth.token_ids(81, n, synth.N_VOCAB)
    got, kinds = _forward(device_layer("ds4_hash"), x, ids=ids)
    _check("ds4_hash", lay, got, x, kinds, "hash n=7", ids=ids)


def test_small_path_errors():
    dev = device_layer("ds4")
    x = m.to_device_x(synth.activations(90, 9, 4096))
    out = torch.zeros((9, 4096), dtype=torch.float32, device="cuda")
    dev.set_path(m.PATH_SMALL)
    try:
        for n in (1, 9):
            with pytest.raises(m.Ds4MoeError) as ei:
                dev.forward(x[:n], out[:n])
            assert ei.value.code == m.EUNSUPPORTED
    finally:
        dev.set_path(m.PATH_AUTO)
    # fp32 activations: no small-batch path on this layer
    with pytest.raises(m.Ds4MoeError) as ei:
        device_layer("tiny").set_path(m.PATH_SMALL)
    assert ei.value.code == m.EUNSUPPORTED
    assert not out.abs().any()
