"""MI355X-native 2-bit routed-MoE block (ds4 / DeepSeek-V4-Flash shapes).

All compute lives in ``libds4moe.so``: hand-written HIP kernels for gfx950
behind the C ABI declared in ``include/ds4moe.h``.  This module is a thin
ctypes binding with the same entry points: it only marshals torch device
tensors and streams (torch is used for device memory and streams) and raises
when the library returns an error.  There is no fallback: without the built
library every call raises.
"""
from __future__ import annotations

import ctypes
from pathlib import Path
from typing import Optional

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "libds4moe.so"

OK, EINVAL, ENOMEM, EHIP, EUNSUPPORTED, EPOISONED = 0, -1, -2, -3, -4, -5
F32, BF16 = 0, 1
FMT_Q2, FMT_Q4 = 0, 1
PATH_AUTO, PATH_GEMV, PATH_GEMM, PATH_SMALL = 0, 1, 2, 3
SMALL_MAX_TOKENS = 8
ABI_VERSION = 4
TIMING_KINDS = ("route", "gateup_routed", "gateup_shared", "down_routed", "down_shared", "gemm_gateup_routed",
                "gemm_down_routed", "fused", "gemm_prep", "gemm_gateup_shared", "gemm_down_shared",
                "q4_gateup_routed", "q4_down_routed", "cache", "small_gateup", "small_down")

SYMBOLS = ("ds4moe_create", "ds4moe_route", "ds4moe_forward", "ds4moe_set_path", "ds4moe_dequantize",
           "ds4moe_rmsnorm", "ds4moe_forward_stack", "ds4moe_timing_enable", "ds4moe_timing_read",
           "ds4moe_last_routing", "ds4moe_status", "ds4moe_set_wait_limit", "ds4moe_forward_static",
           "ds4moe_route_ids", "ds4moe_forward_ids", "ds4moe_forward_stack_ids", "ds4moe_cache_stats",
           "ds4moe_cache_slots", "ds4moe_debug_gemm_b",
           "ds4moe_destroy", "ds4moe_last_error")


class Ds4MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"ds4moe error {code}: {msg}")
        self.code = code


class Desc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("n_embd", ctypes.c_int32), ("n_ff", ctypes.c_int32),
                ("n_expert", ctypes.c_int32), ("top_k", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("router", ctypes.c_void_p), ("router_bias", ctypes.c_void_p), ("gate", ctypes.c_void_p),
                ("up", ctypes.c_void_p), ("down", ctypes.c_void_p), ("codebook", ctypes.c_void_p),
                ("sh_gate", ctypes.c_void_p), ("sh_up", ctypes.c_void_p), ("sh_down", ctypes.c_void_p),
                ("expert_format", ctypes.c_int32), ("hash_table", ctypes.c_void_p), ("n_vocab", ctypes.c_int64),
                ("expert_cache_slots", ctypes.c_int32)]


_lib = None


def load_library(path: Optional[Path] = None) -> ctypes.CDLL:
    """Load libds4moe.so.  torch is imported first so that the library binds to
    the same HIP runtime as torch's tensors and streams."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    import torch  # noqa: F401  (HIP runtime shared with torch)
    p = Path(path) if path else LIB_PATH
    if not p.exists():
        raise RuntimeError(f"{p} is not built; run __graft_entry__.build() or "
                           "python -m bit_quantized_moe_renorm_amd.build")
    L = ctypes.CDLL(str(p))
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.ds4moe_create.argtypes = [ctypes.POINTER(Desc), P, ctypes.POINTER(P)]
    L.ds4moe_route.argtypes = [P, P, i32, P, P, P, P, P]
    L.ds4moe_forward.argtypes = [P, P, i32, P, P]
    L.ds4moe_set_path.argtypes = [P, i32]
    L.ds4moe_dequantize.argtypes = [P, i32, i32, P, P]
    L.ds4moe_rmsnorm.argtypes = [P, i32, i32, ctypes.c_double, P, P]
    L.ds4moe_forward_stack.argtypes = [P, i32, P, i32, ctypes.c_double, P, P]
    L.ds4moe_timing_enable.argtypes = [P, i32]
    L.ds4moe_timing_read.argtypes = [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    L.ds4moe_last_routing.argtypes = [P, i32, P, P, P, P, P]
    L.ds4moe_status.argtypes = [P]
    L.ds4moe_set_wait_limit.argtypes = [P, i32, i32]
    L.ds4moe_forward_static.argtypes = [P, P, i32, P, P]
    L.ds4moe_route_ids.argtypes = [P, P, P, i32, P, P, P, P, P]
    L.ds4moe_forward_ids.argtypes = [P, P, P, i32, P, P]
    L.ds4moe_forward_stack_ids.argtypes = [P, i32, P, P, i32, ctypes.c_double, P, P]
    L.ds4moe_debug_gemm_b.argtypes = [P, i32, i32, P, P]
    L.ds4moe_cache_stats.argtypes = [P, ctypes.POINTER(ctypes.c_int64), P]
    L.ds4moe_cache_slots.argtypes = [P, ctypes.POINTER(ctypes.c_int32), P]
    L.ds4moe_destroy.argtypes = [P]
    L.ds4moe_last_error.restype = ctypes.c_char_p
    for name in SYMBOLS:
        if name != "ds4moe_last_error":
            getattr(L, name).restype = ctypes.c_int
    if path is None:
        _lib = L
    return L


def _check(rc: int):
    if rc != OK:
        raise Ds4MoeError(rc, load_library().ds4moe_last_error().decode())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_tensor(name, t, dtype, shape, device=None):
    """Raise before a raw pointer crosses the ABI: the library trusts sizes."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


class MoELayer:
    """One MoE layer resident on the GPU (a ``ds4moe_t`` handle).

    ``weights`` holds device tensors in the canonical block layout:
    router fp32 [NE, E], router_bias fp32 [NE] or None, gate/up uint8
    [NE, F, E/256, 66], down uint8 [NE, E, F/256, 84], codebook (host, 256
    uint16 values), sh_gate/sh_up/sh_down bf16 or None; with ``fmt`` "q4"
    (weights["fmt"]) gate, up and down are uint8 [..., 144] Q4_K-style blocks;
    ``hash_table`` (int32 [n_vocab, top_k] on the GPU, or None) makes it a
    hash-routed layer, whose calls take the tokens' ids.  ``cache_slots`` > 0 keeps
    the routed experts in pinned host memory with that many of them in an HBM cache.
    """

    def __init__(self, spec, weights: dict, max_tokens: int, act_dtype: int = BF16, stream=None,
                 cache_slots: int = 0):
        import numpy as np
        L = load_library()
        cb = np.ascontiguousarray(weights["codebook"], dtype=np.uint16)
        self._cb = cb
        fmt = FMT_Q4 if weights.get("fmt", "q2") == "q4" else FMT_Q2
        tab = weights.get("hash_table")
        d = Desc(ABI_VERSION, spec.n_embd, spec.n_ff, spec.n_expert, spec.top_k,
                 1 if weights.get("sh_gate") is not None else 0, max_tokens, act_dtype,
                 _ptr(weights["router"]), _ptr(weights.get("router_bias")), _ptr(weights["gate"]),
                 _ptr(weights["up"]), _ptr(weights["down"]), cb.ctypes.data,
                 _ptr(weights.get("sh_gate")), _ptr(weights.get("sh_up")), _ptr(weights.get("sh_down")), fmt,
                 _ptr(tab), 0 if tab is None else tab.shape[0], cache_slots)
        h = ctypes.c_void_p()
        _check(L.ds4moe_create(ctypes.byref(d), _stream(stream), ctypes.byref(h)))
        self.h = h
        self.spec = spec
        self.max_tokens = max_tokens
        self.act_dtype = act_dtype
        self.fmt = fmt
        self.hashed = tab is not None
        self.cache_slots = cache_slots

    def close(self):
        if getattr(self, "h", None):
            load_library().ds4moe_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_path(self, path: int):
        _check(load_library().ds4moe_set_path(self.h, path))

    def _x_dtype(self):
        import torch
        return torch.bfloat16 if self.act_dtype == BF16 else torch.float32

    def _check_x(self, x):
        import torch
        if not isinstance(x, torch.Tensor) or x.dim() != 2:
            raise ValueError("x: expected a 2-D torch tensor [n_tok, n_embd]")
        _check_tensor("x", x, self._x_dtype(), (x.shape[0], self.spec.n_embd))
        return x.shape[0]

    def _check_ids(self, ids, n, dev):
        import torch
        if ids is not None:
            _check_tensor("token_ids", ids, torch.int32, (n,), dev)
        return ids

    def forward(self, x, out, stream=None, ids=None):
        """out += MoE(x) (x [n, E] of the handle's activation dtype, out [n, E] fp32, both on the GPU);
        ``ids`` (int32 [n] on the GPU) are the tokens' ids, which a hash-routed layer needs."""
        import torch
        n = self._check_x(x)
        _check_tensor("out", out, torch.float32, (n, self.spec.n_embd), x.device)
        L = load_library()
        if ids is None:
            _check(L.ds4moe_forward(self.h, _ptr(x), n, _ptr(out), _stream(stream)))
        else:
            self._check_ids(ids, n, x.device)
            _check(L.ds4moe_forward_ids(self.h, _ptr(x), _ptr(ids), n, _ptr(out), _stream(stream)))

    def forward_static(self, x, out, stream=None):
        """out += MoE(x) for 1..4 tokens with the library's static scratch (allocates nothing)."""
        import torch
        n = self._check_x(x)
        _check_tensor("out", out, torch.float32, (n, self.spec.n_embd), x.device)
        _check(load_library().ds4moe_forward_static(self.h, _ptr(x), n, _ptr(out), _stream(stream)))

    def _routing_buffers(self, n, dev):
        import torch
        k, NE = self.spec.top_k, self.spec.n_expert
        idx = torch.empty((n, k), dtype=torch.int32, device=dev)
        w = torch.empty((n, k), dtype=torch.float32, device=dev)
        off = torch.empty((NE + 1,), dtype=torch.int32, device=dev)
        tok = torch.empty((max(n * k, 1),), dtype=torch.int32, device=dev)
        return idx, w, off, tok

    def route(self, x, stream=None, ids=None):
        """Returns (idx int32 [n,k], w fp32 [n,k], offsets int32 [NE+1], tokens int32 [n*k]);
        ``ids`` as for ``forward``."""
        n = self._check_x(x)
        idx, w, off, tok = self._routing_buffers(n, x.device)
        L = load_library()
        if ids is None:
            _check(L.ds4moe_route(self.h, _ptr(x), n, _ptr(idx), _ptr(w), _ptr(off), _ptr(tok), _stream(stream)))
        else:
            self._check_ids(ids, n, x.device)
            _check(L.ds4moe_route_ids(self.h, _ptr(x), _ptr(ids), n, _ptr(idx), _ptr(w), _ptr(off), _ptr(tok),
                                      _stream(stream)))
        return idx, w, off, tok[: n * self.spec.top_k]

    def last_routing(self, n, stream=None):
        """The routing of the latest forward/route call on this layer (n = its token count),
        as (idx, w, offsets, tokens) like ``route``."""
        import torch
        idx, w, off, tok = self._routing_buffers(n, torch.device("cuda", torch.cuda.current_device()))
        _check(load_library().ds4moe_last_routing(self.h, n, _ptr(idx), _ptr(w), _ptr(off), _ptr(tok),
                                                  _stream(stream)))
        return idx, w, off, tok[: n * self.spec.top_k]

    def status(self) -> int:
        """OK, or EPOISONED once a bounded wait of an earlier call gave up (no synchronisation)."""
        return load_library().ds4moe_status(self.h)

    def set_wait_limit(self, max_polls: int, force_expire: bool = False):
        """Test hook: polls before a bounded wait gives up (0 = default); force_expire makes
        every wait give up."""
        _check(load_library().ds4moe_set_wait_limit(self.h, max_polls, 1 if force_expire else 0))

    def dequantize(self, expert: int, which: int, stream=None):
        """fp32 matrix decoded from the library's repacked layout (0 gate, 1 up, 2 down)."""
        import torch
        s = self.spec
        shape = (s.n_ff, s.n_embd) if which < 2 else (s.n_embd, s.n_ff)
        dst = torch.empty(shape, dtype=torch.float32, device="cuda")
        _check(load_library().ds4moe_dequantize(self.h, expert, which, _ptr(dst), _stream(stream)))
        return dst

    def cache_stats(self, stream=None):
        """HBM expert cache counters: dict(calls, hits, misses, bytes) (synchronises)."""
        v = (ctypes.c_int64 * 4)()
        _check(load_library().ds4moe_cache_stats(self.h, v, _stream(stream)))
        return dict(calls=v[0], hits=v[1], misses=v[2], bytes=v[3])

    def cache_slots_held(self, stream=None):
        """The expert each HBM cache slot holds (-1: empty), as a list (synchronises)."""
        v = (ctypes.c_int32 * self.cache_slots)()
        _check(load_library().ds4moe_cache_slots(self.h, v, _stream(stream)))
        return list(v)

    def debug_gemm_b(self, expert: int, which: int, stream=None):
        """The matrix as the grouped GEMMs feed it to the MFMAs (fp16 values as fp32)."""
        import torch
        s = self.spec
        shape = (s.n_ff, s.n_embd) if which < 2 else (s.n_embd, s.n_ff)
        dst = torch.empty(shape, dtype=torch.float32, device="cuda")
        _check(load_library().ds4moe_debug_gemm_b(self.h, expert, which, _ptr(dst), _stream(stream)))
        return dst

    def timing_enable(self, on: bool = True):
        _check(load_library().ds4moe_timing_enable(self.h, 1 if on else 0))

    def timing_read(self):
        ms = (ctypes.c_double * len(TIMING_KINDS))()
        cnt = (ctypes.c_int64 * len(TIMING_KINDS))()
        _check(load_library().ds4moe_timing_read(self.h, ms, cnt))
        return {TIMING_KINDS[i]: (ms[i], cnt[i]) for i in range(len(TIMING_KINDS)) if cnt[i]}


def rmsnorm(h, eps: float = 1e-6, out=None, stream=None):
    """bf16 RMSNorm (unit gain) of fp32 h [n, E] on the GPU."""
    import torch
    n, E = h.shape
    _check_tensor("h", h, torch.float32, (n, E))
    if out is None:
        out = torch.empty((n, E), dtype=torch.bfloat16, device=h.device)
    _check_tensor("out", out, torch.bfloat16, (n, E), h.device)
    _check(load_library().ds4moe_rmsnorm(_ptr(h), n, E, eps, _ptr(out), _stream(stream)))
    return out


def forward_stack(layers, h, eps: float = 1e-6, x=None, stream=None, ids=None):
    """For each layer in order: x = RMSNorm(h), h += MoE(x), all enqueued by
    one library call (h fp32 [n, E] on the GPU, updated in place; x optional
    bf16 [n, E] scratch; ``ids`` int32 [n] on the GPU, the tokens' ids, needed
    when a layer is hash-routed).  Returns h."""
    import torch
    n, E = h.shape
    _check_tensor("h", h, torch.float32, (n, E))
    if x is None:
        x = torch.empty((n, E), dtype=torch.bfloat16, device=h.device)
    _check_tensor("x", x, torch.bfloat16, (n, E), h.device)
    # a closed layer passes NULL, which the library rejects (DS4MOE_EINVAL)
    hs = (ctypes.c_void_p * len(layers))(*[lay.h.value if lay.h else None for lay in layers])
    if ids is None:
        _check(load_library().ds4moe_forward_stack(hs, len(layers), _ptr(h), n, eps, _ptr(x), _stream(stream)))
    else:
        _check_tensor("token_ids", ids, torch.int32, (n,), h.device)
        _check(load_library().ds4moe_forward_stack_ids(hs, len(layers), _ptr(h), _ptr(ids), n, eps, _ptr(x),
                                                       _stream(stream)))
    return h


def upload_layer(layer, device="cuda"):
    """Copy a host ``synth.Layer`` to device tensors in the canonical layout."""
    import numpy as np
    import torch

    def t(a, dtype=None):
        if a is None:
            return None
        x = torch.from_numpy(np.ascontiguousarray(a))
        if dtype is not None:
            x = x.view(dtype)
        return x.to(device)

    return dict(router=t(layer.router), router_bias=t(layer.router_bias), gate=t(layer.gate), up=t(layer.up),
                down=t(layer.down), codebook=layer.codebook, fmt=getattr(layer, "fmt", "q2"),
                sh_gate=t(None if layer.sh_gate is None else layer.sh_gate.view(np.int16), torch.bfloat16),
                sh_up=t(None if layer.sh_up is None else layer.sh_up.view(np.int16), torch.bfloat16),
                sh_down=t(None if layer.sh_down is None else layer.sh_down.view(np.int16), torch.bfloat16),
                hash_table=t(getattr(layer, "hash_table", None)))


def to_device_ids(ids_np, device="cuda"):
    """Token ids (int32 numpy) as a device tensor."""
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).to(device)


def to_device_x(x_np, device="cuda"):
    """Activations from synth (uint16 bf16 bits or fp32) as a device tensor."""
    import numpy as np
    import torch
    if x_np.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32)).to(device)
