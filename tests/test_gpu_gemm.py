"""GPU parity of the batched (grouped MFMA GEMM) path against the CPU oracle,
through the C ABI.

The batched path rounds activations to fp16 for the routed experts (x and the
SwiGLU output h) and keeps the shared expert exact up to fp32 accumulation, so
its error is a few fp16 roundings averaged over thousands of terms: the bar is
max|gpu - ref| / max|ref| <= 2e-3.  Each test also logs the measured error.
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


def _run(dev, x_np, path, out0=None, chunk=None):
    x = m.to_device_x(x_np)
    n = x.shape[0]
    out = torch.zeros((n, x.shape[1]), dtype=torch.float32, device="cuda")
    if out0 is not None:
        out.copy_(torch.from_numpy(out0))
    dev.set_path(path)
    step = chunk or n
    for t0 in range(0, n, step):
        dev.forward(x[t0:t0 + step], out[t0:t0 + step])
    torch.cuda.synchronize()
    dev.set_path(m.PATH_AUTO)
    return out.cpu().numpy()


def test_gemm_tiny_small_batch():
    lay = host_layer("tiny")
    x = synth.activations(0, 4, 256, bf16=False)
    got = _run(device_layer("tiny"), x, m.PATH_GEMM)
    ref, _, _ = oracle.forward(lay, x)
    err = rel_err(got, ref)
    log(f"[gpu] gemm tiny n=4 rel err {err:.3e}")
    assert err <= REL_TOL


def test_gemm_tiny_multi_chunk_experts():
    """300 tokens over 8 experts (top-2): every expert holds more than one
    chunk of 64 slots, with a ragged last chunk."""
    lay = host_layer("tiny")
    x = synth.activations(3, 300, 256, bf16=False)
    got = _run(device_layer("tiny", 512), x, m.PATH_GEMM)
    ref, idx, _ = oracle.forward(lay, x)
    counts = np.bincount(idx.ravel(), minlength=8)
    log(f"[gpu] tiny 300 tokens, slots per expert {counts.tolist()}")
    assert counts.max() > 64
    err = rel_err(got, ref)
    log(f"[gpu] gemm tiny n=300 rel err {err:.3e}")
    assert err <= REL_TOL


@pytest.mark.parametrize("n", [2, 3, 5, 8, 16, 32])
def test_gemm_zipf_batches(n):
    """Decode batches under a Zipf-skewed router bias (AUTO takes the GEMM path for bf16 batches).
    2 and 3 tokens split the GEMMs' K range 8 ways, 5 tokens 4 ways, 8 and more not at all
    (routed) while the shared expert still splits."""
    lay = host_layer("ds4_zipf")
    x = synth.activations(2, n, 4096)
    got = _run(device_layer("ds4_zipf"), x, m.PATH_AUTO)
    ref, _, _ = oracle.forward(lay, x)
    err = rel_err(got, ref)
    log(f"[gpu] gemm zipf n={n} rel err {err:.3e}")
    assert err <= REL_TOL


def test_gemm_matches_gemv_path():
    """The two device paths agree on the same 4 tokens (GEMV keeps fp32 activations)."""
    dev = device_layer("ds4")
    x = synth.activations(4, 4, 4096)
    a = _run(dev, x, m.PATH_GEMV)
    b = _run(dev, x, m.PATH_GEMM)
    err = rel_err(b, a)
    log(f"[gpu] gemm vs gemv rel diff {err:.3e}")
    assert err <= REL_TOL


def test_gemm_accumulates_into_residual():
    lay = host_layer("ds4")
    x = synth.activations(5, 24, 4096)
    r = synth.residual(6, 24, 4096)
    got = _run(device_layer("ds4"), x, m.PATH_GEMM, out0=r)
    ref, _, _ = oracle.forward(lay, x)
    assert rel_err(got - r, ref) <= REL_TOL


_PREFILL = {}


def _prefill_outputs():
    """2048-token prefill in one call and in chunks of 512 (cached)."""
    if not _PREFILL:
        dev = device_layer("ds4", 2048)
        x = synth.activations(1, 2048, 4096)
        log("[gpu] prefill 2048 one call")
        _PREFILL["x"] = x
        _PREFILL["one"] = _run(dev, x, m.PATH_AUTO)
        log("[gpu] prefill 2048 in chunks of 512")
        _PREFILL["chunked"] = _run(dev, x, m.PATH_AUTO, chunk=512)
    return _PREFILL


def test_gemm_prefill_2048_sampled_tokens():
    """Full-size prefill, checked against the oracle on a sample of tokens
    (first, last, chunk edges and a seeded spread)."""
    p = _prefill_outputs()
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 511, 512, 1023, 1024, 2046, 2047],
                                     rng.choice(2048, 22, replace=False)])).astype(np.int32)
    ref, _, _ = oracle.forward(host_layer("ds4"), p["x"], rows=rows)
    err = rel_err(p["one"][rows], ref)
    log(f"[gpu] prefill 2048: {len(rows)} sampled tokens, rel err {err:.3e}")
    assert err <= REL_TOL
    assert np.all(np.isfinite(p["one"]))


def test_gemm_prefill_chunked_512_matches():
    """Prefill in chunks of 512 tokens gives the single-call result (same
    arithmetic per token; only the order of the output atomics differs)."""
    p = _prefill_outputs()
    err = rel_err(p["chunked"], p["one"])
    log(f"[gpu] prefill 512-chunks vs one call rel diff {err:.3e}")
    assert err <= 1e-5
