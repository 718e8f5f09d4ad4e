"""Plain CPU oracle for the top-k routed MoE FFN layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``, never by the product library,
which shares no code with it.  The arithmetic lives in ``moe_oracle.c``
(double precision, token by token, in the order the method defines); this
module only marshals numpy arrays into it.

Storage conventions of the arrays passed in:
  * f32  -> ``np.float32``
  * bf16 -> ``np.uint16`` bit patterns
  * MXFP4 -> ``np.uint8`` codes (two per byte, even element in the low nibble)
    plus ``np.uint8`` E8M0 scales, one per 32 elements along K.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

F32, BF16, MXFP4 = 0, 1, 2
DTYPES = {"f32": F32, "bf16": BF16, "mxfp4": MXFP4}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math: IEEE double throughout)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fopenmp", "-fPIC",
            "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [
        ("H", ctypes.c_int32), ("E", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("I", ctypes.c_int32), ("I_shared", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
        ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
        ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
        ("w_down", ctypes.c_void_p),
        ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p),
        ("s_down", ctypes.c_void_p),
        ("sh_gate", ctypes.c_void_p), ("sh_up", ctypes.c_void_p),
        ("sh_down", ctypes.c_void_p),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.or_bf16_to_f64.restype = ctypes.c_double
        lib.or_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.or_e2m1_value.restype = ctypes.c_double
        lib.or_e2m1_value.argtypes = [ctypes.c_uint8]
        lib.or_e8m0_value.restype = ctypes.c_double
        lib.or_e8m0_value.argtypes = [ctypes.c_uint8]
        lib.or_decode.argtypes = [P, P, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, P]
        lib.or_route.argtypes = [P, P, ctypes.c_int, P, P, P, P]
        lib.or_topk_margin.argtypes = [P, P, ctypes.c_int, P, P]
        lib.or_permute.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P, P]
        lib.or_forward.argtypes = [P, P, ctypes.c_int, P, P, P, P]
        lib.or_set_threads.argtypes = [ctypes.c_int]
        lib.or_max_threads.argtypes = []
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("oracle %s failed with code %d" % (what, rc))


@dataclass
class Layer:
    """One MoE layer's weights as host arrays (see module docstring)."""
    H: int
    E: int
    top_k: int
    I: int
    act: str
    w: str
    router_w: np.ndarray
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray
    router_bias: Optional[np.ndarray] = None
    s_gate: Optional[np.ndarray] = None
    s_up: Optional[np.ndarray] = None
    s_down: Optional[np.ndarray] = None
    I_shared: int = 0
    sh_gate: Optional[np.ndarray] = None
    sh_up: Optional[np.ndarray] = None
    sh_down: Optional[np.ndarray] = None

    def _struct(self) -> _Problem:
        p = _Problem()
        p.H, p.E, p.top_k, p.I = self.H, self.E, self.top_k, self.I
        p.I_shared = self.I_shared
        p.act_dtype, p.w_dtype = DTYPES[self.act], DTYPES[self.w]
        p.router_w = _ptr(self.router_w)
        if self.router_bias is not None:
            assert self.router_bias.dtype == np.float32
        p.router_bias = _ptr(self.router_bias)
        p.w_gate, p.w_up, p.w_down = _ptr(self.w_gate), _ptr(self.w_up), _ptr(self.w_down)
        p.s_gate, p.s_up, p.s_down = _ptr(self.s_gate), _ptr(self.s_up), _ptr(self.s_down)
        p.sh_gate, p.sh_up, p.sh_down = _ptr(self.sh_gate), _ptr(self.sh_up), _ptr(self.sh_down)
        return p


def _tokens(tokens, T):
    if tokens is None:
        return None, T
    tk = np.ascontiguousarray(tokens, dtype=np.int32)
    assert tk.ndim == 1 and (tk.size == 0 or (tk.min() >= 0 and tk.max() < T))
    return tk, tk.size


def route(layer: Layer, x: np.ndarray, tokens=None):
    """Top-k indices [n,k] int32, weights [n,k] f64 and logits [n,E] f64."""
    tk, n = _tokens(tokens, x.shape[0])
    idx = np.empty((n, layer.top_k), np.int32)
    w = np.empty((n, layer.top_k), np.float64)
    logits = np.empty((n, layer.E), np.float64)
    p = layer._struct()
    _check(_load().or_route(ctypes.byref(p), _ptr(x), n, _ptr(tk), _ptr(idx),
                            _ptr(w), _ptr(logits)), "route")
    return idx, w, logits


def topk_margin(layer: Layer, x: np.ndarray, tokens=None) -> np.ndarray:
    """Per token, the smallest neighbour gap among the k+1 largest logits."""
    tk, n = _tokens(tokens, x.shape[0])
    gap = np.empty(n, np.float64)
    p = layer._struct()
    _check(_load().or_topk_margin(ctypes.byref(p), _ptr(x), n, _ptr(tk), _ptr(gap)),
           "topk_margin")
    return gap


def permute(idx: np.ndarray, E: int):
    """Stable grouping of (t, j) pairs by expert: counts, offsets, row_src."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    n, k = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    row_src = np.empty(n * k, np.int32)
    _check(_load().or_permute(n, k, E, _ptr(idx), _ptr(counts), _ptr(offsets),
                              _ptr(row_src)), "permute")
    return counts, offsets, row_src


def forward(layer: Layer, x: np.ndarray, tokens=None):
    """y [n,H] f64 for the listed tokens (all if None), with idx and w."""
    tk, n = _tokens(tokens, x.shape[0])
    y = np.empty((n, layer.H), np.float64)
    idx = np.empty((n, layer.top_k), np.int32)
    w = np.empty((n, layer.top_k), np.float64)
    p = layer._struct()
    _check(_load().or_forward(ctypes.byref(p), _ptr(x), n, _ptr(tk), _ptr(y),
                              _ptr(idx), _ptr(w)), "forward")
    return y, idx, w


def decode(a: np.ndarray, dtype: str, N: int, K: int, scales=None) -> np.ndarray:
    """Exact values of an [N, K] matrix stored as f32, bf16 or MXFP4."""
    out = np.empty((N, K), np.float64)
    _check(_load().or_decode(_ptr(a), _ptr(scales), DTYPES[dtype], N, K, _ptr(out)),
           "decode")
    return out


def bf16_to_f64(v: int) -> float:
    return _load().or_bf16_to_f64(v)


def e2m1_value(code: int) -> float:
    return _load().or_e2m1_value(code)


def e8m0_value(s: int) -> float:
    return _load().or_e8m0_value(s)


def set_threads(n: int) -> None:
    """OpenMP threads the oracle uses (timing only: results do not depend on it)."""
    _check(_load().or_set_threads(int(n)), "set_threads")


def max_threads() -> int:
    return int(_load().or_max_threads())
