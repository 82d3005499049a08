"""The C ABI's failure handling on the GPU: bounded waits that give up are
reported to the host and poison the handle, graph capture is refused, and
misaligned or mistyped buffers are rejected before anything is enqueued.

The wait-expiry tests force the condition from the host (the test hook makes
every bounded wait look for a tag that no producer writes, with a limit of a
few polls), so every kernel still runs to its end."""
import numpy as np
import pytest

from bit_quantized_moe_renorm_amd import synth
from gpu_common import host_layer, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_moe_renorm_amd as m  # noqa: E402


def _fresh(kind, max_tokens=8):
    """A handle of its own (these tests poison it)."""
    lay = host_layer(kind)
    act = m.F32 if kind == "tiny" else m.BF16
    return m.MoELayer(lay.spec, m.upload_layer(lay), max_tokens=max_tokens, act_dtype=act)


@pytest.mark.parametrize("kind,n", [("tiny", 1), ("ds4", 1), ("ds4", 3)])
def test_expired_wait_poisons_handle(kind, n):
    """n = 1: the fused decode kernel's routing and h waits; n = 3: the
    small-batch router's tail.  The call's output (or routing weights) turns
    NaN, and the handle reports DS4MOE_EPOISONED from then on."""
    dev = _fresh(kind)
    E = dev.spec.n_embd
    x = m.to_device_x(synth.activations(0 if kind == "tiny" else 1, n, E, bf16=kind != "tiny"))
    out = torch.zeros((n, E), dtype=torch.float32, device="cuda")
    # a healthy call first
    dev.forward(x, out)
    torch.cuda.synchronize()
    assert dev.status() == m.OK and bool(torch.isfinite(out).all())
    log(f"[gpu] forcing every bounded wait to expire: {kind} n={n}")
    dev.set_wait_limit(4, force_expire=True)
    out.zero_()
    dev.forward(x, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    if n == 1:
        assert np.isnan(got[0, 0]), "the fused decode did not poison its output"
    else:
        assert not np.all(np.isfinite(got)), "the small-batch path did not poison its output"
    assert dev.status() == m.EPOISONED
    with pytest.raises(m.Ds4MoeError) as ei:
        dev.forward(x, out)
    assert ei.value.code == m.EPOISONED
    with pytest.raises(m.Ds4MoeError) as ei:
        dev.route(x)
    assert ei.value.code == m.EPOISONED
    dev.close()


def test_graph_capture_is_refused():
    dev = _fresh("tiny")
    x = m.to_device_x(synth.activations(0, 2, 256, bf16=False))
    out = torch.zeros((2, 256), dtype=torch.float32, device="cuda")
    bufs = dev._routing_buffers(2, x.device)          # nothing is allocated during the capture
    L = m.load_library()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g.capture_begin()
        try:
            sp = m._stream(s)
            rc_fwd = L.ds4moe_forward(dev.h, x.data_ptr(), 2, out.data_ptr(), sp)
            rc_route = L.ds4moe_route(dev.h, x.data_ptr(), 2, *[b.data_ptr() for b in bufs], sp)
        finally:
            g.capture_end()
    torch.cuda.synchronize()
    assert (rc_fwd, rc_route) == (m.EUNSUPPORTED, m.EUNSUPPORTED)
    assert b"captured" in L.ds4moe_last_error()
    # the handle is still usable outside the capture
    dev.forward(x, out)
    torch.cuda.synchronize()
    assert dev.status() == m.OK and bool(torch.isfinite(out).all())
    dev.close()


def test_misaligned_and_mistyped_buffers():
    dev = _fresh("ds4")
    E = dev.spec.n_embd
    buf = torch.zeros(2 * E + 16, dtype=torch.bfloat16, device="cuda")
    x_bad = buf[1:1 + E].view(1, E)           # contiguous, 2 bytes off alignment
    out = torch.zeros((1, E), dtype=torch.float32, device="cuda")
    with pytest.raises(m.Ds4MoeError) as ei:
        dev.forward(x_bad, out)
    assert ei.value.code == m.EINVAL and "aligned" in str(ei.value)
    obuf = torch.zeros(E + 4, dtype=torch.float32, device="cuda")
    x = torch.zeros((1, E), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.Ds4MoeError) as ei:
        dev.forward(x, obuf[1:1 + E].view(1, E))
    assert ei.value.code == m.EINVAL and "aligned" in str(ei.value)
    # the binding refuses what the library cannot check: dtype, shape, device, layout
    with pytest.raises(TypeError):
        dev.forward(x.float(), out)
    with pytest.raises(TypeError):
        dev.forward(x, out.double())
    with pytest.raises(ValueError):
        dev.forward(torch.zeros((1, E // 2), dtype=torch.bfloat16, device="cuda"), out)
    with pytest.raises(ValueError):
        dev.forward(x.cpu(), out)
    with pytest.raises(ValueError):
        dev.forward(torch.zeros((1, 2 * E), dtype=torch.bfloat16, device="cuda")[:, ::2], out)
    # last_routing needs the token count of the latest call
    dev.forward(x, out)
    with pytest.raises(m.Ds4MoeError) as ei:
        dev.last_routing(2)
    assert ei.value.code == m.EINVAL
    torch.cuda.synchronize()
    assert dev.status() == m.OK
    dev.close()


def test_create_out_of_device_memory():
    """With nearly all device memory taken, create fails with DS4MOE_ENOMEM
    and releases what it had allocated: once the memory is back, the same
    description creates a working layer."""
    lay = host_layer("ds4")
    w = m.upload_layer(lay)
    torch.cuda.synchronize()
    free, _ = torch.cuda.mem_get_info()
    log(f"[gpu] taking {free / 2**30:.1f} GiB of device memory, all but 256 MiB")
    hog = []
    left = free - (256 << 20)
    chunk = 16 << 30
    while left > (64 << 20):
        n = min(chunk, left)
        try:
            hog.append(torch.empty(n, dtype=torch.uint8, device="cuda"))
            left -= n
        except RuntimeError:
            chunk //= 2
            if chunk < (64 << 20):
                break
    with pytest.raises(m.Ds4MoeError) as ei:
        m.MoELayer(lay.spec, w, max_tokens=64, act_dtype=m.BF16)
    assert ei.value.code == m.ENOMEM
    del hog
    torch.cuda.empty_cache()
    dev = m.MoELayer(lay.spec, w, max_tokens=64, act_dtype=m.BF16)
    x = m.to_device_x(synth.activations(1, 1, 4096))
    out = torch.zeros((1, 4096), dtype=torch.float32, device="cuda")
    dev.forward(x, out)
    torch.cuda.synchronize()
    assert dev.status() == m.OK and bool(torch.isfinite(out).all())
    dev.close()
