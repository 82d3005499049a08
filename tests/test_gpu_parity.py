"""GPU parity against the CPU oracle, through the C ABI.

Bit-exact: decoded weights, routed expert indices, per-expert token lists.
Within tolerance: renormalised routing weights (fp32 ulps) and block outputs
(max|gpu - ref| / max|ref| <= 2e-3).
"""
import numpy as np
import pytest

import oracle
from bit_quantized_moe_renorm_amd import synth
from gpu_common import FUSED_TOL, GEMV_TOL, REL_TOL, device_layer, host_layer, log, rel_err, tie_split_tokens

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_moe_renorm_amd as m  # noqa: E402


# ------------------------------------------------------------------ dequantisation
@pytest.mark.parametrize("kind,experts", [("tiny", list(range(8))), ("ds4", [0, 97, 255])])
def test_dequant_bitwise(kind, experts):
    lay = host_layer(kind)
    dev = device_layer(kind)
    for e in experts:
        for which, name in enumerate(("gate", "up", "down")):
            log(f"[gpu] dequant {kind} expert {e} {name}")
            got = dev.dequantize(e, which).cpu().numpy()
            ref = oracle.dequant_matrix(lay, e, name)
            assert got.shape == ref.shape
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (kind, e, name)


# ------------------------------------------------------------------ routing
def _check_route(kind, x_np, dev, lay):
    x = m.to_device_x(x_np)
    idx, w, off, tok = dev.route(x)
    torch.cuda.synchronize()
    lg, ridx, rw, rw64 = oracle.route(x_np, lay.router, lay.router_bias, lay.spec.top_k)
    roff, rtok = oracle.bucket(ridx, lay.spec.n_expert)
    idx, w, off, tok = idx.cpu().numpy(), w.cpu().numpy(), off.cpu().numpy(), tok.cpu().numpy()
    bad = np.nonzero(np.any(idx != ridx, axis=1))[0]
    if len(bad):
        t = bad[0]
        srt = np.sort(lg[t])[::-1]
        log(f"[gpu] route mismatch token {t}: gpu {idx[t]} ref {ridx[t]} gap6/7 {srt[5] - srt[6]}")
    assert np.array_equal(idx, ridx), kind
    assert np.array_equal(off, roff), kind
    assert np.array_equal(tok, rtok), kind
    assert np.max(np.abs(w.astype(np.float64) - rw64)) <= 2.5e-7, kind
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)


def test_route_tiny():
    lay = host_layer("tiny")
    _check_route("tiny", synth.activations(0, 4, 256, bf16=False), device_layer("tiny"), lay)


@pytest.mark.parametrize("n", [1, 3, 16, 64])
def test_route_ds4_decode(n):
    lay = host_layer("ds4")
    log(f"[gpu] route ds4 n={n}")
    _check_route("ds4", synth.activations(1, n, 4096), device_layer("ds4"), lay)


@pytest.mark.parametrize("n", [8, 16, 32])
def test_route_zipf_batches(n):
    lay = host_layer("ds4_zipf")
    log(f"[gpu] route ds4 zipf n={n}")
    _check_route("zipf", synth.activations(1, n, 4096), device_layer("ds4_zipf"), lay)


def test_route_prefill_2048():
    lay = host_layer("ds4")
    log("[gpu] route ds4 n=2048")
    _check_route("prefill", synth.activations(1, 2048, 4096), device_layer("ds4", 2048), lay)


@pytest.mark.parametrize("n", [65, 300])
def test_route_ds4_batched(n):
    """Above 64 bf16 tokens the router runs as MFMA estimates plus exact fp64
    logits for the candidates; the result must not change."""
    lay = host_layer("ds4")
    log(f"[gpu] route ds4 batched n={n}")
    _check_route("batched", synth.activations(3, n, 4096), device_layer("ds4", 2048), lay)


def test_route_batched_exact_ties():
    """Identical router rows in pairs: equal logits everywhere, so the estimates
    cannot separate the twins and the lower expert index must win."""
    lay = host_layer("ds4_ties")
    log("[gpu] route ds4 with tied router rows, n=256")
    x = synth.activations(4, 256, 4096)
    _check_route("ties", x, device_layer("ds4_ties", 256), lay)
    _, ridx, _, _ = oracle.route(x, lay.router, lay.router_bias, lay.spec.top_k)
    # the tie rule is exercised: some token takes both experts of a pair
    assert any(len(set(r // 2)) < len(r) for r in ridx)


def _tie_inputs(n):
    x = synth.activations(21, 160, 4096)
    t = tie_split_tokens("ds4_ties_half", x, n)
    assert len(t) == n, "not enough tokens whose top-k boundary splits a tied pair"
    return x[t]


@pytest.mark.parametrize("n", [2, 8, 32])
def test_route_small_batch_tie_boundary(n):
    """The 2..64-token router (tagged top-k in the last workgroup of each token
    tile): every token's k-th expert has an exactly tied twin outside the
    selection, so only the lower-index rule picks between them."""
    lay = host_layer("ds4_ties_half")
    log(f"[gpu] route tie boundary n={n}")
    _check_route("ties_half", _tie_inputs(n), device_layer("ds4_ties_half"), lay)


def _check_last_routing(dev, lay, x_np, n):
    idx, w, off, tok = dev.last_routing(n)
    torch.cuda.synchronize()
    _, ridx, _, rw64 = oracle.route(x_np, lay.router, lay.router_bias, lay.spec.top_k)
    roff, rtok = oracle.bucket(ridx, lay.spec.n_expert)
    idx, w, off, tok = idx.cpu().numpy(), w.cpu().numpy(), off.cpu().numpy(), tok.cpu().numpy()
    assert np.array_equal(idx, ridx), (idx, ridx)
    assert np.array_equal(off, roff) and np.array_equal(tok, rtok)
    assert np.max(np.abs(w.astype(np.float64) - rw64)) <= 2.5e-7


def test_fused_decode_tie_boundary():
    """One-token forward (the fused decode kernel, which takes its own top-k):
    its routing, read back with last_routing, is bit-exact against the oracle
    on tokens whose k-th expert has a tied twin, and the output (the twins'
    weights differ) is within the fused path's tolerance."""
    lay = host_layer("ds4_ties_half")
    dev = device_layer("ds4_ties_half")
    xs = _tie_inputs(8)
    for i in range(len(xs)):
        got = _forward(dev, xs[i:i + 1], m.PATH_AUTO)
        _check_last_routing(dev, lay, xs[i:i + 1], 1)
        ref, _, _ = oracle.forward(lay, xs[i:i + 1])
        err = rel_err(got, ref)
        log(f"[gpu] fused tie-boundary token {i}: rel err {err:.3e}")
        assert err <= FUSED_TOL


def test_fused_decode_routing_matches_oracle():
    """The fused decode kernel's own routing on ordinary tokens (no ties)."""
    lay = host_layer("ds4")
    dev = device_layer("ds4")
    x = synth.activations(1, 6, 4096, start=200)
    for t in range(6):
        _forward(dev, x[t:t + 1], m.PATH_AUTO)
        _check_last_routing(dev, lay, x[t:t + 1], 1)


def test_batched_forward_tie_boundary():
    """8 tie-boundary tokens through the batched path (small-batch router, then
    the grouped GEMMs): routing bit-exact, output within the bar."""
    lay = host_layer("ds4_ties_half")
    dev = device_layer("ds4_ties_half")
    xs = _tie_inputs(8)
    got = _forward(dev, xs, m.PATH_AUTO)
    _check_last_routing(dev, lay, xs, 8)
    ref, _, _ = oracle.forward(lay, xs)
    err = rel_err(got, ref)
    log(f"[gpu] batched tie-boundary n=8 rel err {err:.3e}")
    assert err <= REL_TOL


def test_route_empty_and_errors():
    dev = device_layer("tiny")
    x = torch.zeros((0, 256), device="cuda")
    idx, w, off, tok = dev.route(x)     # n_tok == 0: nothing enqueued
    assert idx.numel() == 0
    with pytest.raises(m.Ds4MoeError) as ei:
        dev.forward(torch.zeros((65, 256), device="cuda"), torch.zeros((65, 256), device="cuda"))
    assert ei.value.code == m.EINVAL


# ------------------------------------------------------------------ block output, GEMV path
def _forward(dev, x_np, path=m.PATH_AUTO, out0=None):
    x = m.to_device_x(x_np)
    out = torch.zeros((x.shape[0], x.shape[1]), dtype=torch.float32, device="cuda")
    if out0 is not None:
        out.copy_(torch.from_numpy(out0))
    dev.set_path(path)
    dev.forward(x, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_forward_tiny_gemv():
    lay = host_layer("tiny")
    x = synth.activations(0, 4, 256, bf16=False)
    got = _forward(device_layer("tiny"), x, m.PATH_GEMV)
    ref, _, _ = oracle.forward(lay, x)
    err = rel_err(got, ref)
    log(f"[gpu] tiny gemv rel err {err:.3e}")
    assert err <= GEMV_TOL


@pytest.mark.parametrize("n", [1, 2, 4])
def test_forward_ds4_gemv(n):
    lay = host_layer("ds4")
    x = synth.activations(1, n, 4096, start=10)
    log(f"[gpu] ds4 gemv n={n}")
    got = _forward(device_layer("ds4"), x, m.PATH_GEMV)
    ref, _, _ = oracle.forward(lay, x)
    err = rel_err(got, ref)
    log(f"[gpu] ds4 gemv n={n} rel err {err:.3e}")
    # one token takes the fused decode launch
    assert err <= REL_TOL and err <= (FUSED_TOL if n == 1 else GEMV_TOL)


def test_forward_tiny_fused_decode():
    """n_tok = 1 takes the single persistent launch."""
    lay = host_layer("tiny")
    x = synth.activations(0, 4, 256, bf16=False)
    dev = device_layer("tiny")
    for t in range(4):
        got = _forward(dev, x[t:t + 1], m.PATH_AUTO)
        ref, _, _ = oracle.forward(lay, x[t:t + 1])
        err = rel_err(got, ref)
        log(f"[gpu] tiny fused token {t} rel err {err:.3e}")
        assert err <= FUSED_TOL


def test_forward_ds4_fused_decode_many_tokens():
    """Consecutive single-token calls (the counters reset between launches)."""
    lay = host_layer("ds4")
    dev = device_layer("ds4")
    x = synth.activations(1, 24, 4096, start=100)
    got = np.stack([_forward(dev, x[t:t + 1], m.PATH_AUTO)[0] for t in range(24)])
    ref, _, _ = oracle.forward(lay, x)
    err = rel_err(got, ref)
    log(f"[gpu] ds4 fused 24 tokens rel err {err:.3e}")
    assert err <= REL_TOL and err <= FUSED_TOL


def test_forward_fused_zipf_bias():
    lay = host_layer("ds4_zipf")
    dev = device_layer("ds4_zipf")
    x = synth.activations(1, 4, 4096, start=7)
    got = np.stack([_forward(dev, x[t:t + 1], m.PATH_AUTO)[0] for t in range(4)])
    ref, _, _ = oracle.forward(lay, x)
    assert rel_err(got, ref) <= FUSED_TOL


def test_forward_accumulates_into_residual():
    lay = host_layer("ds4")
    x = synth.activations(1, 1, 4096, start=3)
    r = synth.residual(5, 1, 4096)
    got = _forward(device_layer("ds4"), x, m.PATH_GEMV, out0=r)  # one token: the fused decode
    ref, _, _ = oracle.forward(lay, x)
    assert rel_err(got - r, ref) <= FUSED_TOL
    got2 = _forward(device_layer("ds4"), np.concatenate([x, x]), m.PATH_GEMV, out0=np.concatenate([r, r]))
    assert rel_err(got2[1] - r[0], ref[0]) <= GEMV_TOL


def test_forward_gemv_rejects_large_batches():
    dev = device_layer("ds4")
    dev.set_path(m.PATH_GEMV)
    x = torch.zeros((5, 4096), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((5, 4096), device="cuda")
    with pytest.raises(m.Ds4MoeError) as ei:
        dev.forward(x, out)
    assert ei.value.code == m.EUNSUPPORTED
    dev.set_path(m.PATH_AUTO)


# ------------------------------------------------------------------ RMSNorm
@pytest.mark.parametrize("n_tok,n_embd", [(33, 4096), (1, 4096), (3, 3072), (5, 1000), (2, 256)])
def test_rmsnorm_matches_oracle(n_tok, n_embd):
    """Bit-exact against the oracle: rows of 1024 k floats take the vector
    kernel, the others the strided one."""
    h = (synth.residual(7, n_tok, n_embd) * 3).astype(np.float32)
    got = m.rmsnorm(torch.from_numpy(h).cuda()).cpu().view(torch.int16).numpy().view(np.uint16)
    ref, _ = oracle.rmsnorm(h, 1e-6)
    assert np.array_equal(got, ref)
