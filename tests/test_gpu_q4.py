"""GPU parity of layers whose routed experts are Q4_K-style blocks (the q4
model's format) against the CPU oracle, through the C ABI.

Decoded weights bit-exact; routing bit-exact; outputs within the GEMV
tolerance: the kernels take bf16 x exactly and fp32 inputs to 22 bits (an
fp16 high and low part), the weights enter the fp16 dot products as the
exact numbers 1 + q/64, and subtracting the staged input sum afterwards costs
about 3 bits of the fp32 result, so the error stays near fp32 rounding."""
import functools

import numpy as np
import pytest

import oracle
from bit_quantized_moe_renorm_amd import synth
from gpu_common import GEMV_TOL, REL_TOL, log, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_moe_renorm_amd as m  # noqa: E402


@functools.lru_cache(maxsize=None)
def _host(kind):
    if kind == "tiny":
        return synth.make_layer(synth.TINY, seed=0, fmt="q4")
    return synth.make_layer(synth.DS4, seed=1, fmt="q4")


_DEV = {}


def _dev(kind):
    if kind not in _DEV:
        lay = _host(kind)
        log(f"[gpu] create q4 layer {kind}")
        act = m.F32 if kind == "tiny" else m.BF16
        _DEV[kind] = m.MoELayer(lay.spec, m.upload_layer(lay), max_tokens=16, act_dtype=act)
    return _DEV[kind]


@pytest.mark.parametrize("kind,experts", [("tiny", list(range(8))), ("ds4", [0, 131, 255])])
def test_q4_dequant_bitwise(kind, experts):
    lay, dev = _host(kind), _dev(kind)
    for e in experts:
        for which, name in enumerate(("gate", "up", "down")):
            got = dev.dequantize(e, which).cpu().numpy()
            ref = oracle.dequant_matrix(lay, e, name)
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (kind, e, name)


def _run(dev, x_np, static=False):
    x = m.to_device_x(x_np)
    out = torch.zeros((x.shape[0], x.shape[1]), dtype=torch.float32, device="cuda")
    (dev.forward_static if static else dev.forward)(x, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("n", [1, 3, 4, 9])
def test_q4_tiny_forward(n):
    lay, dev = _host("tiny"), _dev("tiny")
    x = synth.activations(0, n, 256, bf16=False)
    got = _run(dev, x)
    ref, ridx, _ = oracle.forward(lay, x)
    err = rel_err(got, ref)
    log(f"[gpu] q4 tiny n={n} rel err {err:.3e}")
    assert err <= GEMV_TOL


@pytest.mark.parametrize("n", [1, 2, 4, 7])
def test_q4_ds4_forward(n):
    """1..4 tokens: one chunk; 7 (an MTP verification shape): two chunks."""
    lay, dev = _host("ds4"), _dev("ds4")
    x = synth.activations(1, n, 4096, start=40)
    got = _run(dev, x)
    ref, ridx, _ = oracle.forward(lay, x)
    err = rel_err(got, ref)
    log(f"[gpu] q4 ds4 n={n} rel err {err:.3e}")
    assert err <= GEMV_TOL
    if n <= 4:
        idx = dev.last_routing(n)[0].cpu().numpy()
        assert np.array_equal(idx, ridx)


def test_q4_forward_static_and_route():
    lay, dev = _host("ds4"), _dev("ds4")
    x = synth.activations(1, 3, 4096, start=90)
    ref, ridx, _ = oracle.forward(lay, x)
    got = _run(dev, x, static=True)
    assert rel_err(got, ref) <= GEMV_TOL
    idx, w, off, tok = dev.route(m.to_device_x(x))
    assert np.array_equal(idx.cpu().numpy(), ridx)
    with pytest.raises(m.Ds4MoeError) as ei:
        dev.set_path(m.PATH_GEMM)
    assert ei.value.code == m.EUNSUPPORTED
    assert REL_TOL >= GEMV_TOL


def _wide_range(x32):
    """Seeded activations with a different power-of-two magnitude per 64-value
    chunk (2^-20 .. 2^20), an all-zero chunk 0 and one large value in chunk 1:
    the Q4_K kernels stage their inputs per chunk under a power-of-two scale,
    so this covers empty chunks, both ends of the scale and a chunk whose
    values span 2^25."""
    x = np.array(x32, dtype=np.float32, copy=True)
    nch = x.shape[1] // 64
    for c in range(nch):
        x[:, 64 * c:64 * c + 64] *= np.float32(2.0 ** (((7 * c) % 41) - 20))
    x[:, 0:64] = 0.0
    x[:, 64:128] *= np.float32(2.0 ** -12)
    x[:, 69] = np.float32(3.0e4)
    return x


@pytest.mark.parametrize("kind,n", [("tiny", 1), ("tiny", 3), ("ds4", 1), ("ds4", 2)])
def test_q4_wide_range_inputs(kind, n):
    lay, dev = _host(kind), _dev(kind)
    E = lay.spec.n_embd
    if kind == "tiny":
        x = _wide_range(synth.activations(0, n, E, bf16=False, start=20))
    else:
        x32 = synth.bf16_bits_to_f32(synth.activations(1, n, E, start=120))
        x = synth.f32_to_bf16_bits(_wide_range(x32))
    got = _run(dev, x)
    ref, ridx, _ = oracle.forward(lay, x)
    err = rel_err(got, ref)
    log(f"[gpu] q4 {kind} wide-range n={n} rel err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= GEMV_TOL
