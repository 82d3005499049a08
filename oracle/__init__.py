"""CPU oracle for ds4's 2-bit routed-MoE block — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``oracle.c`` (plain C, fp64,
OpenMP) through ctypes and shares no code with the HIP library.

Every function here is pinned by ``-m "not gpu"`` tests (round trips through an
independent encoder, invariants, brute force, dense SwiGLU via numpy).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "oracle.c"
_LIB = _HERE / "liboracle.so"
_lib = None


def build(force: bool = True) -> Path:
    """Compile liboracle.so with gcc -O2 (no fast-math) and OpenMP."""
    if force or not _LIB.exists():
        tmp = _LIB.with_suffix(".so.tmp")
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
                        str(_SRC), "-o", str(tmp), "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not _LIB.exists():
            build(force=False)
        L = ctypes.CDLL(str(_LIB))
        P = ctypes.c_void_p
        i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.oracle_dequant_iq2.argtypes = [P, i64, P, P]
        L.oracle_dequant_q2k.argtypes = [P, i64, P]
        L.oracle_dequant_q4k.argtypes = [P, i64, P]
        L.oracle_route.argtypes = [P, i32, i64, i32, P, P, i32, i32, P, P, P, P]
        L.oracle_route.restype = i32
        L.oracle_bucket.argtypes = [P, i64, i32, i32, P, P]
        L.oracle_forward.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, i32, P, i64,
                                     P, P, i64, P, P, P]
        L.oracle_route_hashed.argtypes = [P, i32, i64, i32, P, P, i32, i32, P, P, i64, P, P, P, P]
        L.oracle_route_hashed.restype = i32
        L.oracle_forward.restype = i32
        L.oracle_rmsnorm.argtypes = [P, i64, i32, f64, P, P]
        L.oracle_num_threads.restype = i32
        L.oracle_set_num_threads.argtypes = [i32]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    """OpenMP threads for later calls (results do not depend on it)."""
    lib().oracle_set_num_threads(int(n))


def dequant_iq2(blocks: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """Decode IQ2-style blocks ``[..., 66]`` to fp32 ``[..., 256]``."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    assert b.shape[-1] == 66
    n = b.size // 66
    out = np.empty(b.shape[:-1] + (256,), dtype=np.float32)
    cb = np.ascontiguousarray(codebook, dtype=np.uint16)
    assert cb.shape == (256,)
    lib().oracle_dequant_iq2(_p(b), n, _p(cb), _p(out))
    return out


def dequant_q2k(blocks: np.ndarray) -> np.ndarray:
    """Decode Q2_K-style blocks ``[..., 84]`` to fp32 ``[..., 256]``."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    assert b.shape[-1] == 84
    n = b.size // 84
    out = np.empty(b.shape[:-1] + (256,), dtype=np.float32)
    lib().oracle_dequant_q2k(_p(b), n, _p(out))
    return out


def dequant_q4k(blocks: np.ndarray) -> np.ndarray:
    """Decode Q4_K-style blocks ``[..., 144]`` to fp32 ``[..., 256]``."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    assert b.shape[-1] == 144
    n = b.size // 144
    out = np.empty(b.shape[:-1] + (256,), dtype=np.float32)
    lib().oracle_dequant_q4k(_p(b), n, _p(out))
    return out


def _fmt(layer) -> int:
    return 1 if getattr(layer, "fmt", "q2") == "q4" else 0


def dequant_matrix(layer, expert: int, which: str) -> np.ndarray:
    """fp32 matrix of one routed expert: gate/up ``[n_ff, n_embd]``, down ``[n_embd, n_ff]``."""
    if _fmt(layer):
        blk = getattr(layer, which)[expert]
        return dequant_q4k(blk).reshape(blk.shape[0], -1)
    if which in ("gate", "up"):
        blk = getattr(layer, which)[expert]
        return dequant_iq2(blk, layer.codebook).reshape(blk.shape[0], -1)
    blk = layer.down[expert]
    return dequant_q2k(blk).reshape(blk.shape[0], -1)


def _x(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, 1
    assert x.dtype == np.float32
    return x, 0


def route(x, router, bias, top_k):
    """Returns (logits fp32 [n, NE], idx int32 [n, k], w fp32 [n, k], w64 fp64 [n, k])."""
    x, isbf = _x(x)
    n, E = x.shape
    router = np.ascontiguousarray(router, dtype=np.float32)
    NE = router.shape[0]
    bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    logits = np.empty((n, NE), np.float32)
    idx = np.empty((n, top_k), np.int32)
    w = np.empty((n, top_k), np.float32)
    w64 = np.empty((n, top_k), np.float64)
    rc = lib().oracle_route(_p(x), isbf, n, E, _p(router), _p(bias), NE, top_k, _p(logits),
                            _p(idx), _p(w), _p(w64))
    assert rc == 0, rc
    return logits, idx, w, w64


def route_hashed(x, router, bias, top_k, token_ids, table):
    """Hash routing: experts from ``table[token_ids[t]]`` (slot order), weights the
    softmax renormalised over them.  Returns (logits, idx, w, w64) like ``route``."""
    x, isbf = _x(x)
    n, E = x.shape
    router = np.ascontiguousarray(router, dtype=np.float32)
    NE = router.shape[0]
    bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    ids = np.ascontiguousarray(token_ids, dtype=np.int32)
    tab = np.ascontiguousarray(table, dtype=np.int32)
    assert ids.shape == (n,) and tab.shape[1] == top_k
    logits = np.empty((n, NE), np.float32)
    idx = np.empty((n, top_k), np.int32)
    w = np.empty((n, top_k), np.float32)
    w64 = np.empty((n, top_k), np.float64)
    rc = lib().oracle_route_hashed(_p(x), isbf, n, E, _p(router), _p(bias), NE, top_k, _p(ids), _p(tab),
                                   tab.shape[0], _p(logits), _p(idx), _p(w), _p(w64))
    assert rc == 0, rc
    return logits, idx, w, w64


def bucket(idx: np.ndarray, n_expert: int):
    """Per-expert token lists: (offsets int32 [NE+1], tokens int32 [n*k])."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    n, k = idx.shape
    offsets = np.empty(n_expert + 1, np.int32)
    tokens = np.empty(n * k, np.int32)
    lib().oracle_bucket(_p(idx), n, k, n_expert, _p(offsets), _p(tokens))
    return offsets, tokens


def forward(layer, x, rows=None, token_ids=None):
    """MoE(x) for the tokens in ``rows`` (default all): returns (out fp64 [r, E], idx, w64).
    A hash-routed layer (``layer.hash_table`` set) needs the tokens' ids."""
    x, isbf = _x(x)
    n, E = x.shape
    s = layer.spec
    assert E == s.n_embd
    rows = np.arange(n, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    out = np.empty((len(rows), E), np.float64)
    idx = np.empty((len(rows), s.top_k), np.int32)
    w = np.empty((len(rows), s.top_k), np.float64)
    tab = getattr(layer, "hash_table", None)
    ids = None
    if tab is not None:
        assert token_ids is not None and len(token_ids) == n, "a hash-routed layer needs the token ids"
        tab = np.ascontiguousarray(tab, dtype=np.int32)
        ids = np.ascontiguousarray(token_ids, dtype=np.int32)
    rc = lib().oracle_forward(E, s.n_ff, s.n_expert, s.top_k, _fmt(layer), _p(layer.router), _p(layer.router_bias),
                              _p(layer.gate), _p(layer.up), _p(layer.down), _p(layer.codebook),
                              _p(layer.sh_gate), _p(layer.sh_up), _p(layer.sh_down), _p(x), isbf,
                              _p(rows), len(rows), _p(ids), _p(tab), 0 if tab is None else tab.shape[0],
                              _p(out), _p(idx), _p(w))
    assert rc == 0, rc
    return out, idx, w


def rmsnorm(h: np.ndarray, eps: float = 1e-6):
    """(bf16 bits [n, E], fp64 values [n, E]) of h / sqrt(mean(h^2) + eps)."""
    h = np.ascontiguousarray(h, dtype=np.float32)
    n, E = h.shape
    xb = np.empty((n, E), np.uint16)
    x64 = np.empty((n, E), np.float64)
    lib().oracle_rmsnorm(_p(h), n, E, eps, _p(xb), _p(x64))
    return xb, x64


def stack(layers, h0: np.ndarray, eps: float = 1e-6, token_ids=None):
    """A stack of MoE layers on the residual stream h (fp32 [n, E]).

    Each layer normalises h (RMSNorm with unit gain, ``rmsnorm`` above), runs
    the MoE block on the bf16 result and adds it to h: h <- h + MoE(x), the sum
    in fp64 and stored in fp32, the residual stream's type at the block's
    boundary.  The pages describe the model's hyper-connection mixing rather
    than a per-layer norm for this block; the stack is the plainest one around
    it.  A hash-routed layer (``hash_table`` set) routes by the tokens' ids,
    ``token_ids`` [n].  Returns (h after the last layer, [x_l bf16 bits],
    [idx_l], [logits_l]).
    """
    h = np.ascontiguousarray(h0, dtype=np.float32).copy()
    xs, idxs, logits = [], [], []
    for layer in layers:
        xb, _ = rmsnorm(h, eps)
        if getattr(layer, "hash_table", None) is not None:
            lg, idx, _, _ = route_hashed(xb, layer.router, layer.router_bias, layer.spec.top_k, token_ids,
                                         layer.hash_table)
        else:
            lg, idx, _, _ = route(xb, layer.router, layer.router_bias, layer.spec.top_k)
        y, _, _ = forward(layer, xb, token_ids=token_ids)
        h = (h.astype(np.float64) + y).astype(np.float32)
        xs.append(xb)
        idxs.append(idx)
        logits.append(lg)
    return h, xs, idxs, logits
