"""ds4moe_forward_static (the entry point that allocates nothing: its scratch
is the library's static per-GPU device array) against ds4moe_forward, through
the C ABI, on two calls in a row with the second one smaller."""
import ctypes

import numpy as np
import pytest

from bit_quantized_moe_renorm_amd import synth
from gpu_common import FUSED_TOL, GEMV_TOL, device_layer, log, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_moe_renorm_amd as m  # noqa: E402


def _pair(dev, x_np):
    """(forward_static output, forward output, their routings) for the same x;
    the reference takes the same kernels (the GEMV path for 2..4 tokens)."""
    L = m.load_library()
    x = m.to_device_x(x_np)
    n, E = x.shape
    out_s = torch.zeros((n, E), dtype=torch.float32, device="cuda")
    out_r = torch.zeros((n, E), dtype=torch.float32, device="cuda")
    s = m._stream(None)
    rc = L.ds4moe_forward_static(dev.h, ctypes.c_void_p(x.data_ptr()), n, ctypes.c_void_p(out_s.data_ptr()), s)
    assert rc == m.OK, L.ds4moe_last_error()
    r_s = [t.cpu().numpy() for t in dev.last_routing(n)]
    dev.set_path(m.PATH_GEMV)
    dev.forward(x, out_r)
    dev.set_path(m.PATH_AUTO)
    r_r = [t.cpu().numpy() for t in dev.last_routing(n)]
    torch.cuda.synchronize()
    return out_s.cpu().numpy(), out_r.cpu().numpy(), r_s, r_r


def _check(tag, dev, x_np):
    got, ref, r_s, r_r = _pair(dev, x_np)
    err = rel_err(got, ref)
    log(f"[gpu] forward_static {tag}: n={len(x_np)} rel diff vs forward {err:.3e}")
    assert np.all(np.isfinite(got))
    # same kernels, same inputs: only the order of the fp32 atomics differs
    assert err <= (FUSED_TOL if len(x_np) == 1 else GEMV_TOL)
    for a, b in zip(r_s, r_r):
        assert np.array_equal(a, b) if a.dtype != np.float32 else np.allclose(a, b, rtol=0, atol=0)


def test_forward_static_matches_forward():
    ds4 = device_layer("ds4")
    tiny = device_layer("tiny")
    # DS4 shape: 4 tokens, then 2 (smaller), then one (the fused decode), then 3 again
    x = synth.activations(1, 4, 4096, start=300)
    _check("ds4", ds4, x)
    _check("ds4", ds4, x[:2])
    _check("ds4", ds4, x[3:4])
    _check("ds4", ds4, x[:3])
    # a smaller layer on the same array right after
    xt = synth.activations(0, 4, 256, bf16=False)
    _check("tiny", tiny, xt[:1])
    _check("tiny", tiny, xt[:2])


def test_forward_static_rejects_more_tokens():
    dev = device_layer("ds4")
    L = m.load_library()
    x = torch.zeros((5, 4096), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((5, 4096), dtype=torch.float32, device="cuda")
    rc = L.ds4moe_forward_static(dev.h, ctypes.c_void_p(x.data_ptr()), 5, ctypes.c_void_p(out.data_ptr()),
                                 m._stream(None))
    assert rc == m.EINVAL and b"static scratch" in L.ds4moe_last_error()
    torch.cuda.synchronize()
    assert float(out.abs().sum()) == 0.0
