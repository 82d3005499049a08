"""Inputs whose magnitude changes by up to 2^40 across a token's 64-value
chunks, against the CPU oracle, on the paths that stage activations or h
vectors in fp16 under power-of-two scales: the fused single-token decode (a
scale per 64-value chunk), the small-batch kernels (a scale per token for x,
per vector for h) and the GEMV kernels (fp32 activations, no staging).  The
grouped GEMMs round x to fp16 without a scale (an overflow shows as inf, as
their header states), so they are not given such inputs.

The inputs are the seeded activations scaled by 2^(((7 c) mod 41) - 20) in
chunk c, with an all-zero chunk 0 and a 3e4 value in chunk 1."""
import numpy as np
import pytest

import oracle
from bit_quantized_moe_renorm_amd import synth
from gpu_common import FUSED_TOL, GEMV_TOL, REL_TOL, device_layer, host_layer, log, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_moe_renorm_amd as m  # noqa: E402


def _wide_range(x32):
    x = np.array(x32, dtype=np.float32, copy=True)
    for c in range(x.shape[1] // 64):
        x[:, 64 * c:64 * c + 64] *= np.float32(2.0 ** (((7 * c) % 41) - 20))
    x[:, 0:64] = 0.0
    x[:, 64:128] *= np.float32(2.0 ** -12)
    x[:, 69] = np.float32(3.0e4)
    return x


def _forward(dev, x_np, path):
    dev.set_path(path)
    try:
        x = m.to_device_x(x_np)
        out = torch.zeros((x.shape[0], x.shape[1]), dtype=torch.float32, device="cuda")
        dev.forward(x, out)
        torch.cuda.synchronize()
        return out.cpu().numpy()
    finally:
        dev.set_path(m.PATH_AUTO)


@pytest.mark.parametrize("n,path,tol", [(1, "auto", FUSED_TOL), (7, "auto", REL_TOL), (3, "gemv", GEMV_TOL)])
def test_ds4_wide_range(n, path, tol):
    """DS4 layer, bf16 x: one token (fused decode), 7 (small-batch kernels),
    3 on the GEMV kernels."""
    lay = host_layer("ds4")
    x = synth.f32_to_bf16_bits(_wide_range(synth.bf16_bits_to_f32(synth.activations(1, n, 4096, start=300))))
    got = _forward(device_layer("ds4"), x, m.PATH_AUTO if path == "auto" else m.PATH_GEMV)
    ref, _, _ = oracle.forward(lay, x)
    err = rel_err(got, ref)
    log(f"[gpu] ds4 wide-range n={n} {path} rel err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= tol


@pytest.mark.parametrize("n", [1, 4])
def test_tiny_wide_range(n):
    """Tiny layer, fp32 x: one token (fused decode, x in fp16 high and low
    parts), 4 (GEMV kernels)."""
    lay = host_layer("tiny")
    x = _wide_range(synth.activations(0, n, 256, bf16=False, start=30))
    got = _forward(device_layer("tiny"), x, m.PATH_AUTO)
    ref, _, _ = oracle.forward(lay, x)
    err = rel_err(got, ref)
    log(f"[gpu] tiny wide-range n={n} rel err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= (FUSED_TOL if n == 1 else GEMV_TOL)
