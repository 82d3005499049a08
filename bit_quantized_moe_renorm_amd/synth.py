"""Seeded synthetic inputs for the 2-bit routed-MoE block.

This module only draws random numbers and lays them out as the block's input
tensors.  It holds none of the block's arithmetic (no dequantisation, routing
or matmul), so both the HIP library and the CPU oracle can be fed from it
without sharing any computation.

Shapes follow the model constants printed on "Redis 作者出手！ds4：用 C 语言从零
打造 DeepSeek V4 Flash 本地推理引擎..." (section 2.1: N_EMBD 4096, N_FF_EXP 2048,
N_EXPERT 256, N_EXPERT_USED 6, N_EXPERT_SHARED 1) and the block sizes of its
section 2.3 (66 bytes per 256 weights for the IQ2 codebook format, 84 bytes per
256 weights for the Q2_K format).

Value distributions (all drawn from numpy's PCG64, keyed by (seed, tensor id)):

* activations: N(0, 1), rounded to bf16 (round-to-nearest-even), or kept as
  fp32 for the tiny layer;
* router: N(0, 0.02) fp32, stored expert-major ``[n_expert, n_embd]``;
* shared expert: N(0, 0.02) rounded to bf16;
* every quantised field (codebook index, sign bits, sub-block scales, 2-bit
  quants, scale/min nibbles) is uniform over its bit range;
* the fp16 super-block scales are positive normal fp16 numbers with a uniform
  10-bit mantissa inside one fixed binade: ``[2^-7, 2^-6)`` for the IQ2 ``d``
  and ``[2^-10, 2^-9)`` for the Q2_K ``d`` and ``dmin`` (uniform fp16 bit
  patterns would include NaN and Inf);
* the codebook: 256 entries of 8 two-bit coordinates (uint16, coordinate i in
  bits 2i..2i+1), drawn once from a fixed seed and shared by every layer.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

CODEBOOK_SEED = 0xC0DE_B00C
QK = 256                    # weights per super-block
IQ2_BLOCK_BYTES = 66        # fp16 d + 8 sub-blocks x (4 index bytes + 1 sign/scale word)
Q2K_BLOCK_BYTES = 84        # scales[16] + qs[64] + fp16 d + fp16 dmin
Q4K_BLOCK_BYTES = 144       # fp16 d + fp16 dmin + 16 six-bit scale/min fields + qs[128]

_TID = dict(router=1, router_bias=2, gate=3, up=4, down=5, sh_gate=6, sh_up=7,
            sh_down=8, x=9, codebook=10, h0=11, zipf=12, hash=13, ids=14)
N_VOCAB = 129280            # DS4_N_VOCAB, the model's vocabulary size


def rng_for(seed: int, what: str) -> np.random.Generator:
    """Independent PCG64 stream per (seed, tensor)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), _TID[what]])))


def _raw_bytes(rng: np.random.Generator, n: int) -> np.ndarray:
    words = rng.bit_generator.random_raw((n + 7) // 8)
    return words.view(np.uint8)[:n]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16, nearest-even; returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _fp16_in_binade(rng: np.random.Generator, n: int, exp_field: int) -> np.ndarray:
    """Positive normal fp16 bit patterns with a fixed exponent field and uniform mantissa."""
    mant = rng.integers(0, 1024, size=n, dtype=np.uint16)
    return (np.uint16(exp_field << 10) | mant).astype(np.uint16)


def iq2_blocks(rng: np.random.Generator, n_blocks: int) -> np.ndarray:
    """``n_blocks`` random IQ2-style super-blocks, shape ``[n_blocks, 66]`` uint8.

    Bytes 0-1 hold the fp16 scale ``d`` (little endian), drawn in [2^-7, 2^-6)
    (exponent field 8); bytes 2-65 are uniform random.
    """
    blk = _raw_bytes(rng, n_blocks * IQ2_BLOCK_BYTES).reshape(n_blocks, IQ2_BLOCK_BYTES).copy()
    d = _fp16_in_binade(rng, n_blocks, 8)
    blk[:, 0:2] = d.view(np.uint8).reshape(n_blocks, 2)
    return blk


def q2k_blocks(rng: np.random.Generator, n_blocks: int) -> np.ndarray:
    """``n_blocks`` random Q2_K-style super-blocks, shape ``[n_blocks, 84]`` uint8.

    Bytes 80-81 hold ``d`` and 82-83 ``dmin`` (fp16, little endian), both in
    [2^-10, 2^-9) (exponent field 5); bytes 0-79 are uniform random.
    """
    blk = _raw_bytes(rng, n_blocks * Q2K_BLOCK_BYTES).reshape(n_blocks, Q2K_BLOCK_BYTES).copy()
    dd = _fp16_in_binade(rng, 2 * n_blocks, 5)
    blk[:, 80:84] = dd.view(np.uint8).reshape(n_blocks, 4)
    return blk


def q4k_blocks(rng: np.random.Generator, n_blocks: int) -> np.ndarray:
    """``n_blocks`` random Q4_K-style super-blocks, shape ``[n_blocks, 144]`` uint8.

    Bytes 0-1 hold ``d`` and 2-3 ``dmin`` (fp16, little endian), both in
    [2^-14, 2^-13) (exponent field 1, the smallest normal binade: with 6-bit
    scales and 4-bit quants the weights' spread is then close to the other
    formats'); bytes 4-143 (the scale/min fields and the quants) are uniform
    random.
    """
    blk = _raw_bytes(rng, n_blocks * Q4K_BLOCK_BYTES).reshape(n_blocks, Q4K_BLOCK_BYTES).copy()
    dd = _fp16_in_binade(rng, 2 * n_blocks, 1)
    blk[:, 0:4] = dd.view(np.uint8).reshape(n_blocks, 4)
    return blk


def codebook() -> np.ndarray:
    """The shared 256-entry codebook: uint16 per entry, 2 bits per coordinate."""
    return rng_for(CODEBOOK_SEED, "codebook").integers(0, 1 << 16, size=256, dtype=np.uint16)


@dataclass
class LayerSpec:
    n_embd: int = 4096
    n_ff: int = 2048
    n_expert: int = 256
    top_k: int = 6
    n_shared: int = 1


TINY = LayerSpec(n_embd=256, n_ff=256, n_expert=8, top_k=2, n_shared=1)
DS4 = LayerSpec()


@dataclass
class Layer:
    """Host copy of one MoE layer's weights in the canonical (array-of-blocks) layout.

    * ``router``: fp32 ``[n_expert, n_embd]``; ``router_bias``: fp32 ``[n_expert]`` or None
    * ``gate``, ``up``: uint8 ``[n_expert, n_ff, n_embd/256, 66]`` (rows = output features,
      super-blocks run along the contraction dimension)
    * ``down``: uint8 ``[n_expert, n_embd, n_ff/256, 84]``
    * ``codebook``: uint16 ``[256]``
    * ``sh_gate``, ``sh_up``: bf16 bits ``[n_ff, n_embd]``; ``sh_down``: bf16 bits ``[n_embd, n_ff]``
    * ``fmt``: "q2" (the layout above) or "q4": gate, up and down are all Q4_K-style
      blocks of 144 bytes, ``[n_expert, rows, cols/256, 144]``
    """
    spec: LayerSpec
    seed: int
    router: np.ndarray
    router_bias: Optional[np.ndarray]
    gate: np.ndarray
    up: np.ndarray
    down: np.ndarray
    codebook: np.ndarray
    sh_gate: Optional[np.ndarray]
    sh_up: Optional[np.ndarray]
    sh_down: Optional[np.ndarray]
    extra: dict = field(default_factory=dict)
    fmt: str = "q2"
    hash_table: Optional[np.ndarray] = None   # int32 [n_vocab, top_k] for a hash-routed layer


def zipf_router_bias(seed: int, n_expert: int, s: float = 1.1) -> np.ndarray:
    """Router bias ``-s * ln(r_e)`` with ``r`` a seeded permutation of the ranks 1..n_expert.

    Added to the logits, it skews expert popularity toward a Zipf(s) law.
    """
    ranks = rng_for(seed, "zipf").permutation(n_expert) + 1
    return (-s * np.log(ranks.astype(np.float64))).astype(np.float32)


def make_layer(spec: LayerSpec, seed: int, zipf_bias: bool = False, shared: bool = True, fmt: str = "q2") -> Layer:
    E, F, NE = spec.n_embd, spec.n_ff, spec.n_expert
    assert E % QK == 0 and F % QK == 0 and fmt in ("q2", "q4")
    router = (rng_for(seed, "router").standard_normal((NE, E)) * 0.02).astype(np.float32)
    bias = zipf_router_bias(seed, NE) if zipf_bias else None
    if fmt == "q4":
        B = Q4K_BLOCK_BYTES
        gate = q4k_blocks(rng_for(seed, "gate"), NE * F * (E // QK)).reshape(NE, F, E // QK, B)
        up = q4k_blocks(rng_for(seed, "up"), NE * F * (E // QK)).reshape(NE, F, E // QK, B)
        down = q4k_blocks(rng_for(seed, "down"), NE * E * (F // QK)).reshape(NE, E, F // QK, B)
    else:
        gate = iq2_blocks(rng_for(seed, "gate"), NE * F * (E // QK)).reshape(NE, F, E // QK, IQ2_BLOCK_BYTES)
        up = iq2_blocks(rng_for(seed, "up"), NE * F * (E // QK)).reshape(NE, F, E // QK, IQ2_BLOCK_BYTES)
        down = q2k_blocks(rng_for(seed, "down"), NE * E * (F // QK)).reshape(NE, E, F // QK, Q2K_BLOCK_BYTES)
    if shared and spec.n_shared:
        sg = f32_to_bf16_bits((rng_for(seed, "sh_gate").standard_normal((F, E)) * 0.02).astype(np.float32))
        su = f32_to_bf16_bits((rng_for(seed, "sh_up").standard_normal((F, E)) * 0.02).astype(np.float32))
        sd = f32_to_bf16_bits((rng_for(seed, "sh_down").standard_normal((E, F)) * 0.02).astype(np.float32))
    else:
        sg = su = sd = None
    return Layer(spec, seed, router, bias, gate, up, down, codebook(), sg, su, sd, fmt=fmt)


def hash_table(seed: int, n_vocab: int, n_expert: int, top_k: int) -> np.ndarray:
    """Per-token-id expert table of a hash-routed layer, int32 ``[n_vocab, top_k]``:
    row v holds top_k distinct experts drawn uniformly (the model's own table
    is part of its weights, which the pages do not give)."""
    rng = rng_for(seed, "hash")
    keys = rng.random((n_vocab, n_expert))
    return np.argsort(keys, axis=1)[:, :top_k].astype(np.int32)


def token_ids(seed: int, n_tok: int, n_vocab: int = N_VOCAB, start: int = 0) -> np.ndarray:
    """Rows ``start .. start+n_tok`` of the seed's uniform token-id stream (int32)."""
    return rng_for(seed, "ids").integers(0, n_vocab, size=start + n_tok, dtype=np.int64)[start:].astype(np.int32)


def activations(seed: int, n_tok: int, n_embd: int, bf16: bool = True, start: int = 0) -> np.ndarray:
    """Rows ``start .. start+n_tok`` of the seed's N(0,1) activation stream.

    Returns bf16 bit patterns (uint16) when ``bf16`` else fp32.  Row ``t`` of
    the stream does not depend on how many rows are requested.
    """
    rows = rng_for(seed, "x").standard_normal((start + n_tok, n_embd), dtype=np.float64)[start:]
    a = rows.astype(np.float32)
    return f32_to_bf16_bits(a) if bf16 else a


def residual(seed: int, n_tok: int, n_embd: int) -> np.ndarray:
    """Initial fp32 residual stream ``h0`` ~ N(0, 1) for a stack of layers."""
    return rng_for(seed, "h0").standard_normal((n_tok, n_embd)).astype(np.float32)


def layer_nbytes(spec: LayerSpec, fmt: str = "q2") -> dict:
    """Stored bytes of one layer's tensors (quantised experts as stored)."""
    E, F, NE = spec.n_embd, spec.n_ff, spec.n_expert
    per_gate = F * (E // QK) * (Q4K_BLOCK_BYTES if fmt == "q4" else IQ2_BLOCK_BYTES)
    per_down = E * (F // QK) * (Q4K_BLOCK_BYTES if fmt == "q4" else Q2K_BLOCK_BYTES)
    return dict(per_expert=2 * per_gate + per_down, gate=per_gate, down=per_down,
                shared=3 * E * F * 2 * spec.n_shared, router=NE * E * 4)
