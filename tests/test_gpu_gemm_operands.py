"""What the grouped GEMMs feed the MFMAs, against the oracle's exact weights.

The routed GEMMs take their 2-bit weights as fp16 B operands
(ds4moe_debug_gemm_b decodes a matrix through the kernels' own operand code):
  IQ2:  the signed level times fp16(d (2 ls + 1) / 64), rounded again in the
        product: |B - w| <= 2^-10 |w| (two roundings of 2^-11, every weight a
        normal fp16 for the synthetic scales);
  Q2_K: fma(q, fp16(d sc), fp16(-dmin m)) in fp16: |B - w| <= 2^-11 (q |d sc|
        + |dmin m| + |w|) (1 + 2^-10) + 3 * 2^-25 (the last term for results
        or minima in fp16's subnormal range).
The bounds follow from the roundings alone, so a wrong index, sign, scale or
K position fails them by orders of magnitude.  The debug kernel also decodes
every IQ2 value with the sign-mask table (the path of one- and two-tile
chunks and of the small-batch kernels) and writes NaN where the two decodes
differ in any bit, which fails the bound.
"""
import numpy as np
import pytest

import oracle
from gpu_common import device_layer, host_layer, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_moe_renorm_amd as m  # noqa: E402


def _q2k_terms(blocks):
    """q |d sc| and |dmin m| per weight from canonical Q2_K blocks [rows, nb, 84]."""
    rows, nb, _ = blocks.shape
    scales = blocks[..., 0:16].astype(np.int64)
    sc, mm = scales & 15, scales >> 4
    qs = blocks[..., 16:80].astype(np.int64)
    q = np.stack([(qs >> (2 * j)) & 3 for j in range(4)], axis=-1).reshape(rows, nb, 256)
    d = blocks[..., 80:82].copy().view(np.float16)[..., 0].astype(np.float64)
    dmin = blocks[..., 82:84].copy().view(np.float16)[..., 0].astype(np.float64)
    dsc = np.repeat(d[..., None] * sc, 16, axis=-1)
    dm = np.repeat(dmin[..., None] * mm, 16, axis=-1)
    return (q * np.abs(dsc)).reshape(rows, nb * 256), np.abs(dm).reshape(rows, nb * 256)


@pytest.mark.parametrize("kind,experts", [("tiny", [0, 5]), ("ds4", [0, 200])])
def test_gemm_b_operands_within_fp16_rounding(kind, experts):
    lay = host_layer(kind)
    dev = device_layer(kind)
    for e in experts:
        for which, name in enumerate(("gate", "up", "down")):
            got = dev.debug_gemm_b(e, which).cpu().numpy().astype(np.float64)
            w = oracle.dequant_matrix(lay, e, name).astype(np.float64)
            assert got.shape == w.shape
            if which < 2:
                bound = 2.0 ** -10 * np.abs(w) * (1 + 2.0 ** -20)
            else:
                qd, dm = _q2k_terms(lay.down[e])
                bound = 2.0 ** -11 * (qd + dm + np.abs(w)) * (1 + 2.0 ** -10) + 3 * 2.0 ** -25
            err = np.abs(got - w)
            worst = float(np.max(err / np.maximum(bound, 1e-300)))
            log(f"[gpu] B operand {kind} expert {e} {name}: max |B - w| / bound = {worst:.3f}, "
                f"{np.count_nonzero(err):d} of {err.size} weights rounded")
            assert np.all(err <= bound), (kind, e, name)
            # the rounding to fp16 does happen (this is the path's stated departure from exact weights)
            assert np.count_nonzero(err) > 0


def test_gemm_b_operand_errors():
    dev = device_layer("tiny")
    with pytest.raises(m.Ds4MoeError):
        dev.debug_gemm_b(8, 0)
    with pytest.raises(m.Ds4MoeError):
        dev.debug_gemm_b(0, 3)
