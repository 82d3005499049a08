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


@pytest.mark.parametrize("n", [2, 3, 4, 5, 7, 8, 16, 32])
def test_gemm_zipf_batches(n):
    """Decode batches under a Zipf-skewed router bias, on the GEMM path (AUTO takes the
    small-batch kernels up to 8 bf16 tokens, the GEMM path beyond).
    2 and 3 tokens split the GEMMs' K range 8 ways, 5 tokens 4 ways, 8 and more not at all
    (routed) while the shared expert still splits.  2..8 tokens are also the shapes of
    speculative (MTP) verification, which scores the last token plus k drafted ones in one
    call ("ds4 深度实战...", section 4.2: the optional MTP download for multi-token
    prediction / speculative decoding); 7 is k = 6."""
    lay = host_layer("ds4_zipf")
    x = synth.activations(2, n, 4096)
    got = _run(device_layer("ds4_zipf"), x, m.PATH_GEMM)
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
    """2048-token prefill in one call and in chunks of 512 (cached), and the
    GEMV kernels' result (exact weights, fp32 activations, 4 tokens per call)."""
    if not _PREFILL:
        dev = device_layer("ds4", 2048)
        x = synth.activations(1, 2048, 4096)
        log("[gpu] prefill 2048 one call")
        _PREFILL["x"] = x
        _PREFILL["one"] = _run(dev, x, m.PATH_AUTO)
        log("[gpu] prefill 2048 in chunks of 512")
        _PREFILL["chunked"] = _run(dev, x, m.PATH_AUTO, chunk=512)
        log("[gpu] prefill 2048 through the GEMV kernels, 4 tokens per call")
        _PREFILL["gemv"] = _run(dev, x, m.PATH_GEMV, chunk=4)
    return _PREFILL


def chunk_edge_rows(x_np, k, n_expert, call=2048, chunk=64):
    """Tokens in the first and the last slot of every chunk of CH_TOK = 64
    slots of every expert's list (the grouped GEMMs' work units, ragged tails
    included), for calls of ``call`` tokens; from the oracle's routing."""
    lay = host_layer("ds4")
    rows = set()
    for c0 in range(0, len(x_np), call):
        _, idx, _, _ = oracle.route(x_np[c0:c0 + call], lay.router, lay.router_bias, k)
        offs, toks = oracle.bucket(idx, n_expert)
        for e in range(n_expert):
            lst = toks[offs[e]:offs[e + 1]]
            for s0 in range(0, len(lst), chunk):
                part = lst[s0:s0 + chunk]
                rows.add(c0 + int(part[0]))
                rows.add(c0 + int(part[-1]))
    return np.array(sorted(rows), dtype=np.int32)


def test_gemm_prefill_2048_every_chunk():
    """Full-size prefill against the oracle on the first and last token of
    every expert's 64-slot chunk (so every work unit of the routed GEMMs,
    with its ragged tail, is checked), in one call and in four calls of 512."""
    p = _prefill_outputs()
    rows = np.union1d(chunk_edge_rows(p["x"], 6, 256), chunk_edge_rows(p["x"], 6, 256, call=512))
    log(f"[gpu] prefill 2048: oracle on {len(rows)} chunk-edge tokens")
    ref, _, _ = oracle.forward(host_layer("ds4"), p["x"], rows=rows)
    err = rel_err(p["one"][rows], ref)
    err512 = rel_err(p["chunked"][rows], ref)
    log(f"[gpu] prefill 2048: rel err {err:.3e} (one call), {err512:.3e} (512-token calls)")
    assert err <= REL_TOL and err512 <= REL_TOL
    assert np.all(np.isfinite(p["one"])) and np.all(np.isfinite(p["chunked"]))


def test_gemm_prefill_2048_all_rows_against_gemv():
    """All 2048 rows against the GEMV kernels (exact dequantised weights and
    fp32 activations; within 1e-5 of the oracle in the GEMV tests), at the
    same bar: a fault confined to some rows of the grouped GEMMs shows here."""
    p = _prefill_outputs()
    err = rel_err(p["one"], p["gemv"])
    err512 = rel_err(p["chunked"], p["gemv"])
    log(f"[gpu] prefill 2048 vs GEMV kernels: rel diff {err:.3e} (one call), {err512:.3e} (512-token calls)")
    assert err <= REL_TOL and err512 <= REL_TOL
