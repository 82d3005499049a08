"""Pins for the oracle's block decoders (CPU only).

None of these retypes the decoder: they use hand-built blocks whose values
were worked out by hand (tests/golden), an independent *encoder* written from
the layout (a bit-position mistake in the decoder is not mirrored by it), and
structural invariants that any correct decoder of the layout must satisfy.
"""
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest

from bit_quantized_moe_renorm_amd import synth

GOLDEN = Path(__file__).parent / "golden"


def _read_golden(name):
    fields = {}
    for line in (GOLDEN / name).read_text().splitlines():
        if not line or line.startswith("#"):
            continue
        key, rest = line.split(" ", 1)
        fields.setdefault(key, []).append(rest)
    return fields


def test_page_constants_match_shapes():
    """The model constants and block sizes printed on the pages fix the DS4 shapes."""
    consts = {}
    for line in (GOLDEN / "ds4_constants.txt").read_text().splitlines():
        if line and not line.startswith("#"):
            k, v = line.split()
            consts[k] = float(v)
    s = synth.DS4
    assert s.n_embd == consts["N_EMBD"] and s.n_ff == consts["N_FF_EXP"]
    assert s.n_expert == consts["N_EXPERT"] and s.top_k == consts["N_EXPERT_USED"]
    assert s.n_shared == consts["N_EXPERT_SHARED"]
    assert synth.QK == consts["QK_K"]
    assert synth.Q2K_BLOCK_BYTES == consts["Q2K_BLOCK_BYTES"]
    assert synth.IQ2_BLOCK_BYTES == consts["IQ2XXS_BLOCK_BYTES"]
    assert abs(synth.IQ2_BLOCK_BYTES * 8 / 256 - consts["IQ2XXS_BPW_APPROX"]) < 0.01
    nb = synth.layer_nbytes(s)
    # one routed expert: gate + up (IQ2) + down (Q2_K), as stored
    assert nb["per_expert"] == 7_077_888
    assert nb["shared"] == 50_331_648


# ---------------------------------------------------------------- hand-built blocks
def test_iq2_handbuilt_golden(oracle_lib):
    g = _read_golden("iq2_handbuilt.txt")
    cb = np.zeros(256, np.uint16)
    for row in g["codebook"]:
        i, v = row.split()
        cb[int(i)] = int(v, 16)
    blk = np.frombuffer(bytes.fromhex(g["block"][0]), np.uint8)
    exp = np.array([int(v) for v in g["expected_x64"][0].split()], np.float64) / 64.0
    got = oracle_lib.dequant_iq2(blk[None], cb)[0]
    assert np.array_equal(got.astype(np.float64), exp)
    # same block with d = 0x2A00 = 3/64 (byte order: low byte first)
    blk2 = blk.copy()
    blk2[0], blk2[1] = 0x00, 0x2A
    got2 = oracle_lib.dequant_iq2(blk2[None], cb)[0]
    assert np.array_equal(got2.astype(np.float64), exp * 3 / 64)


def test_q2k_handbuilt_golden(oracle_lib):
    g = _read_golden("q2k_handbuilt.txt")
    blk = np.frombuffer(bytes.fromhex(g["block"][0]), np.uint8)
    exp = np.array([int(v) for v in g["expected_x2"][0].split()], np.float64) / 2.0
    got = oracle_lib.dequant_q2k(blk[None])[0]
    assert np.array_equal(got.astype(np.float64), exp)


# ---------------------------------------------------------------- independent encoders
def _fp16_bits(v: float) -> int:
    return int(np.array([v], np.float16).view(np.uint16)[0])


def encode_iq2(d: float, ls, idx, signs):
    """Pack one IQ2-style block from field values.

    ls[8] sub-block scales, idx[32] codebook indices, signs[32][8] booleans
    (each group must hold an even number of True: the 8th sign is implied).
    """
    out = bytearray(66)
    out[0:2] = _fp16_bits(d).to_bytes(2, "little")
    for s in range(8):
        word = int(ls[s]) << 28
        for g in range(4):
            grp = 4 * s + g
            bits = signs[grp]
            assert sum(bits) % 2 == 0
            for i in range(7):
                if bits[i]:
                    word |= 1 << (7 * g + i)
            out[2 + 8 * s + g] = int(idx[grp])
        out[2 + 8 * s + 4: 2 + 8 * s + 8] = word.to_bytes(4, "little")
    return np.frombuffer(bytes(out), np.uint8)


def encode_q2k(d: float, dmin: float, sc, m, q):
    out = bytearray(84)
    for s in range(16):
        out[s] = (int(m[s]) << 4) | int(sc[s])
    for i in range(256):
        out[16 + i // 4] |= int(q[i]) << (2 * (i % 4))
    out[80:82] = _fp16_bits(d).to_bytes(2, "little")
    out[82:84] = _fp16_bits(dmin).to_bytes(2, "little")
    return np.frombuffer(bytes(out), np.uint8)


def test_iq2_encoder_roundtrip(oracle_lib):
    """Random field values -> encoder -> oracle; compare with the values the fields denote.

    The codebook levels are read back per coordinate (level set {1,3,5,7}/8) and the
    sub-block scale as (2 ls + 1)/8, and the result is built as an exact rational.
    """
    rng = np.random.default_rng(7)
    levels = [Fraction(1, 8), Fraction(3, 8), Fraction(5, 8), Fraction(7, 8)]
    cb = rng.integers(0, 1 << 16, 256, dtype=np.uint16)
    for trial in range(20):
        d = float(np.float16(rng.uniform(2 ** -7, 2 ** -6)))
        ls = rng.integers(0, 16, 8)
        idx = rng.integers(0, 256, 32)
        signs = []
        for _ in range(32):
            b = [bool(v) for v in rng.integers(0, 2, 7)]
            b.append(sum(b) % 2 == 1)
            signs.append(b)
        blk = encode_iq2(d, ls, idx, signs)
        got = oracle_lib.dequant_iq2(blk[None], cb)[0]
        for grp in range(32):
            s = grp // 4
            entry = int(cb[idx[grp]])
            for i in range(8):
                coord = (entry >> (2 * i)) & 3
                val = Fraction(d) * Fraction(2 * int(ls[s]) + 1, 8) * levels[coord]
                if signs[grp][i]:
                    val = -val
                assert Fraction(float(got[8 * grp + i])) == val, (trial, grp, i)


def test_q2k_encoder_roundtrip(oracle_lib):
    rng = np.random.default_rng(8)
    for trial in range(20):
        d = float(np.float16(rng.uniform(2 ** -10, 2 ** -9)))
        dmin = float(np.float16(rng.uniform(2 ** -10, 2 ** -9)))
        sc = rng.integers(0, 16, 16)
        m = rng.integers(0, 16, 16)
        q = rng.integers(0, 4, 256)
        blk = encode_q2k(d, dmin, sc, m, q)
        got = oracle_lib.dequant_q2k(blk[None])[0]
        for i in range(256):
            val = Fraction(d) * int(sc[i // 16]) * int(q[i]) - Fraction(dmin) * int(m[i // 16])
            assert Fraction(float(got[i])) == val, (trial, i)


def test_q2k_exhaustive_unit_scales(oracle_lib):
    """d = dmin = 1: every (sc, m, q) combination decodes to the integer sc*q - m."""
    blocks, exp = [], []
    for sc in range(16):
        for m in range(16):
            q = np.tile(np.arange(4), 64)
            blocks.append(encode_q2k(1.0, 1.0, [sc] * 16, [m] * 16, q))
            exp.append(sc * q - m)
    got = oracle_lib.dequant_q2k(np.stack(blocks))
    assert np.array_equal(got, np.array(exp, np.float32))


def test_iq2_exhaustive_scale_index_sign(oracle_lib):
    """d = 1: all 16 scales x 256 indices x 128 sign patterns; |w| in 64ths is an odd
    product, the sign set obeys the parity rule, and every stored sign pattern appears."""
    cb = synth.codebook()
    rng = np.random.default_rng(9)
    blocks = []
    meta = []
    for ls in range(16):
        for idx0 in range(0, 256, 32):
            ids = np.arange(idx0, idx0 + 32) % 256
            pat = rng.permutation(128)[:32]
            signs = []
            for p in pat:
                b = [bool((p >> i) & 1) for i in range(7)]
                b.append(sum(b) % 2 == 1)
                signs.append(b)
            blocks.append(encode_iq2(1.0, [ls] * 8, ids, signs))
            meta.append((ls, ids, signs))
    got = oracle_lib.dequant_iq2(np.stack(blocks), cb) * 64.0
    for b, (ls, ids, signs) in enumerate(meta):
        v = got[b].reshape(32, 8)
        for grp in range(32):
            entry = int(cb[ids[grp]])
            mags = [(2 * ls + 1) * (2 * ((entry >> (2 * i)) & 3) + 1) for i in range(8)]
            assert np.array_equal(np.abs(v[grp]), np.array(mags, np.float32))
            assert list(v[grp] < 0) == signs[grp]
            assert (v[grp] < 0).sum() % 2 == 0


# ---------------------------------------------------------------- structural invariants
def test_iq2_invariants(oracle_lib):
    rng = np.random.default_rng(11)
    blk = synth.iq2_blocks(rng, 64)
    cb = synth.codebook()
    base = oracle_lib.dequant_iq2(blk, cb)
    # each 8-weight group has an even number of negatives
    assert np.all((base.reshape(-1, 8) < 0).sum(1) % 2 == 0)
    # flipping stored sign bit i of group g flips exactly weights i and 7 of that group
    for (b, s, g, i) in [(0, 0, 0, 0), (3, 5, 2, 6), (10, 7, 3, 3)]:
        mod = blk.copy()
        bit = 7 * g + i
        mod[b, 2 + 8 * s + 4 + bit // 8] ^= 1 << (bit % 8)
        out = oracle_lib.dequant_iq2(mod, cb)
        diff = np.nonzero(out != base)
        lo = 256 * b + 32 * s + 8 * g
        assert sorted(zip(*diff)) == sorted([(b, 32 * s + 8 * g + i), (b, 32 * s + 8 * g + 7)]), lo
        assert np.array_equal(out[b, 32 * s + 8 * g + i], -base[b, 32 * s + 8 * g + i])
    # changing ls of sub-block s rescales exactly that sub-block by (2ls'+1)/(2ls+1)
    mod = blk.copy()
    old = mod[5, 2 + 8 * 4 + 7] >> 4
    new = (old + 5) % 16
    mod[5, 2 + 8 * 4 + 7] = (mod[5, 2 + 8 * 4 + 7] & 0x0F) | (new << 4)
    out = oracle_lib.dequant_iq2(mod, cb)
    ratio = out[5, 128:160].astype(np.float64) / base[5, 128:160]
    assert np.allclose(ratio, (2 * new + 1) / (2 * old + 1), rtol=0, atol=1e-12)
    mask = np.ones_like(base, bool)
    mask[5, 128:160] = False
    assert np.array_equal(out[mask], base[mask])
    # d = 0 zeroes the block; doubling d (exponent + 1) doubles it
    mod = blk.copy()
    mod[2, 0:2] = 0
    mod[4, 1] += 0x04
    out = oracle_lib.dequant_iq2(mod, cb)
    assert np.all(out[2] == 0)
    assert np.array_equal(out[4], base[4] * 2)
    # codebook entry change only touches the groups that use it
    cb2 = cb.copy()
    k = int(blk[1, 2])
    cb2[k] ^= 0x3
    out = oracle_lib.dequant_iq2(blk, cb2)
    used = np.zeros(base.shape, bool)
    for b in range(64):
        for s in range(8):
            for g in range(4):
                if blk[b, 2 + 8 * s + g] == k:
                    used[b, 32 * s + 8 * g] = True
    assert np.all(out[~used] == base[~used])
    assert np.all(out[used] != base[used])


def test_q2k_invariants(oracle_lib):
    rng = np.random.default_rng(12)
    blk = synth.q2k_blocks(rng, 32)
    base = oracle_lib.dequant_q2k(blk).astype(np.float64)
    d = blk[:, 80:82].copy().view(np.float16).astype(np.float64)
    dmin = blk[:, 82:84].copy().view(np.float16).astype(np.float64)
    # within a 16-weight sub-block, values step by d*sc per quant level: the spread is d*sc*3 at most
    sub = base.reshape(32, 16, 16)
    spread = sub.max(2) - sub.min(2)
    assert np.all(spread <= d * 15 * 3 + 1e-12)
    # dmin = 0 and sc = 0 everywhere -> all zero
    mod = blk.copy()
    mod[:, 82:84] = 0
    mod[:, 0:16] &= 0xF0
    assert np.all(oracle_lib.dequant_q2k(mod) == 0)
    # setting all quants to 0 leaves -dmin*m per sub-block (only the min term survives)
    mod = blk.copy()
    mod[:, 16:80] = 0
    out = oracle_lib.dequant_q2k(mod).astype(np.float64).reshape(32, 16, 16)
    m = (blk[:, 0:16] >> 4).astype(np.float64)
    assert np.array_equal(out, np.broadcast_to((-dmin * m)[:, :, None], out.shape))
    # swapping d and dmin bytes moves the scale between the two terms
    assert np.all(np.isfinite(base))


def test_synth_fields_in_range():
    rng = np.random.default_rng(3)
    b = synth.iq2_blocks(rng, 1000)
    d = b[:, 0:2].copy().view(np.float16).astype(np.float64)
    assert np.all((d >= 2 ** -7) & (d < 2 ** -6))
    q = synth.q2k_blocks(rng, 1000)
    dd = q[:, 80:84].copy().view(np.float16).astype(np.float64)
    assert np.all((dd >= 2 ** -10) & (dd < 2 ** -9))
    # the random fields cover their range
    assert len(np.unique(b[:, 2:])) == 256


def test_dequant_exact_in_fp32(oracle_lib):
    """Random blocks: the fp32 result equals the exact rational value of the fields."""
    rng = np.random.default_rng(13)
    blk = synth.q2k_blocks(rng, 4)
    got = oracle_lib.dequant_q2k(blk)
    for b in range(4):
        d = Fraction(float(blk[b, 80:82].copy().view(np.float16)[0]))
        dmin = Fraction(float(blk[b, 82:84].copy().view(np.float16)[0]))
        for i in range(0, 256, 7):
            sc, m = int(blk[b, i // 16] & 15), int(blk[b, i // 16] >> 4)
            qv = (int(blk[b, 16 + i // 4]) >> (2 * (i % 4))) & 3
            assert Fraction(float(got[b, i])) == d * sc * qv - dmin * m
