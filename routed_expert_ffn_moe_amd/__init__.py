"""Python binding of libmoe.so, the gfx950 routed-expert MoE FFN layer.

Argument marshalling only: torch tensors are passed by device pointer and
every step of the layer runs in the library's HIP kernels.  The functions
carry the names of the C entry points declared in ``include/moe.h``.

The library must have been built (``python -m routed_expert_ffn_moe_amd.build``);
importing the binding does not build it, and every call fails loudly when the
library is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "MOE_F32", "MOE_BF16", "MOE_MXFP4", "MOE_LAYOUT_ROWMAJOR", "MOE_LAYOUT_PACKED", "MOE_OK",
    "MOE_EINVAL", "MOE_EWORKSPACE", "MOE_EUNSUPPORTED", "MOE_EHIP", "MoeError", "moe_shape_t", "moe_weights_t", "make_shape",
    "make_weights", "moe_workspace_bytes", "moe_forward", "moe_forward_noalloc",
    "MOE_NOALLOC_SCRATCH_BYTES", "moe_route", "moe_strerror",
    "moe_last_error", "moe_stage_timing_enable", "moe_stage_timing_read", "moe_pack_bf16",
    "pack_bf16", "moe_pack_mxfp4", "pack_mxfp4", "STAGES", "moe_probe_read", "moe_probe_mfma",
    "moe_probe_gather", "moe_probe_mxfp4",
    "lib_path", "load",
]

MOE_F32, MOE_BF16, MOE_MXFP4 = 0, 1, 2
MOE_LAYOUT_ROWMAJOR, MOE_LAYOUT_PACKED = 0, 1
MOE_OK, MOE_EINVAL, MOE_EWORKSPACE, MOE_EUNSUPPORTED, MOE_EHIP = 0, -1, -2, -3, -4
_DT = {"f32": MOE_F32, "bf16": MOE_BF16, "mxfp4": MOE_MXFP4}

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_HERE, "libmoe.so")


class MoeError(RuntimeError):
    def __init__(self, code: int, detail: str):
        super().__init__("%s (%d): %s" % (moe_strerror(code), code, detail))
        self.code = code


class moe_shape_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "H", "E", "top_k", "I", "I_shared", "chunk_T", "act_dtype", "w_dtype")]


class moe_weights_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("router_w", "router_bias", "w_gate", "w_up", "w_down", "s_gate", "s_up",
                 "s_down", "sh_gate", "sh_up", "sh_down")] + [("layout", ctypes.c_int32)]


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError("libmoe.so is not built: run `python -m routed_expert_ffn_moe_amd.build`")
        # torch ships its own HIP runtime (file libamdhip64.so, soname
        # libamdhip64.so.7).  Loaded first, it is the one libmoe.so binds to.
        # Loaded after libmoe.so, torch would bring a second runtime into the
        # process beside ROCm's, and the two cannot both own the device: the
        # library's calls would then fail with "no ROCm-capable device".
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        lib.moe_workspace_bytes.restype = ctypes.c_size_t
        lib.moe_workspace_bytes.argtypes = [P]
        lib.moe_forward.restype = ctypes.c_int
        lib.moe_forward.argtypes = [P, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.moe_forward_noalloc.restype = ctypes.c_int
        lib.moe_forward_noalloc.argtypes = [P, P, P, P, P, P, P]
        lib.moe_route.restype = ctypes.c_int
        lib.moe_route.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.moe_strerror.restype = ctypes.c_char_p
        lib.moe_strerror.argtypes = [ctypes.c_int]
        lib.moe_last_error.restype = ctypes.c_char_p
        lib.moe_last_error.argtypes = []
        lib.moe_stage_timing_enable.restype = ctypes.c_int
        lib.moe_stage_timing_enable.argtypes = [ctypes.c_int]
        lib.moe_stage_timing_read.restype = ctypes.c_int
        lib.moe_stage_timing_read.argtypes = [P, ctypes.c_int, P]
        lib.moe_pack_bf16.restype = ctypes.c_int
        lib.moe_pack_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P]
        lib.moe_pack_mxfp4.restype = ctypes.c_int
        lib.moe_pack_mxfp4.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P, P, P]
        lib.moe_probe_read.restype = ctypes.c_int
        lib.moe_probe_read.argtypes = [P, ctypes.c_size_t, P]
        lib.moe_probe_mfma.restype = ctypes.c_int
        lib.moe_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, P, P]
        lib.moe_probe_gather.restype = ctypes.c_int
        lib.moe_probe_gather.argtypes = [P, ctypes.c_size_t, ctypes.c_size_t, P, ctypes.c_int,
                                         ctypes.c_int, P]
        lib.moe_probe_mxfp4.restype = ctypes.c_int
        lib.moe_probe_mxfp4.argtypes = [P, P, ctypes.c_size_t, ctypes.c_int, P, P]
        _lib = lib
    return _lib


def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor (None -> NULL; ints pass through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_shape(T, H, E, top_k, I, I_shared=0, chunk_T=0, act="bf16", w="bf16") -> moe_shape_t:
    return moe_shape_t(T, H, E, top_k, I, I_shared, chunk_T, _DT[act], _DT[w])


class _Weights:
    """moe_weights_t plus references keeping the tensors alive."""

    def __init__(self, layout, **tensors):
        self._keep = tensors
        self.c = moe_weights_t(**{k: _ptr(v) for k, v in tensors.items()}, layout=layout)


def _is_packed(t) -> bool:
    return t is not None and getattr(t, "_moe_layout", None) == "packed"


def make_weights(router_w, w_gate, w_up, w_down, router_bias=None, s_gate=None, s_up=None,
                 s_down=None, sh_gate=None, sh_up=None, sh_down=None, layout=None) -> _Weights:
    """The weight struct.  `layout` (MOE_LAYOUT_*) defaults to PACKED when
    every expert matrix given came out of pack_bf16 / pack_mxfp4, else
    ROWMAJOR; the library refuses bf16 / MXFP4 matrices declared ROWMAJOR."""
    if layout is None:
        mats = [m for m in (w_gate, w_up, w_down, sh_gate, sh_up, sh_down) if m is not None]
        layout = MOE_LAYOUT_PACKED if all(_is_packed(m) for m in mats) else MOE_LAYOUT_ROWMAJOR
    return _Weights(layout, router_w=router_w, router_bias=router_bias, w_gate=w_gate, w_up=w_up,
                    w_down=w_down, s_gate=s_gate, s_up=s_up, s_down=s_down, sh_gate=sh_gate,
                    sh_up=sh_up, sh_down=sh_down)


def _check(rc: int):
    if rc != MOE_OK:
        raise MoeError(rc, moe_last_error())


def moe_workspace_bytes(shape: moe_shape_t) -> int:
    return int(load().moe_workspace_bytes(ctypes.byref(shape)))


def moe_forward(shape, weights, x, y, topk_idx, topk_w, ws, ws_bytes=None, stream=None) -> None:
    """y[T,H] and the routing of x[T,H]; asynchronous on `stream`."""
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().moe_forward(ctypes.byref(shape), ctypes.byref(weights.c), _ptr(x), _ptr(y),
                              _ptr(topk_idx), _ptr(topk_w), _ptr(ws), ws_bytes,
                              _stream(stream)))


MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_forward_noalloc(shape, weights, x, y, topk_idx, topk_w, stream=None) -> None:
    """moe_forward on the library's static device scratch (allocates nothing)."""
    _check(load().moe_forward_noalloc(ctypes.byref(shape), ctypes.byref(weights.c), _ptr(x),
                                      _ptr(y), _ptr(topk_idx), _ptr(topk_w), _stream(stream)))


def moe_route(shape, weights, x, topk_idx, topk_w, counts, offsets, row_src, ws, ws_bytes=None,
              stream=None) -> None:
    """Router and permutation of one pass (see include/moe.h)."""
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().moe_route(ctypes.byref(shape), ctypes.byref(weights.c), _ptr(x),
                            _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets),
                            _ptr(row_src), _ptr(ws), ws_bytes, _stream(stream)))


def moe_pack_bf16(E, N, K, w, w_out, stream=None) -> None:
    """Repack row-major bf16 matrices [E, N, K] into the layout moe_forward reads."""
    _check(load().moe_pack_bf16(E, N, K, _ptr(w), _ptr(w_out), _stream(stream)))


def pack_bf16(w, stream=None):
    """Packed copy of a bf16 device tensor [E, N, K] or [N, K]."""
    import torch
    E, N, K = (1, *w.shape) if w.dim() == 2 else w.shape
    out = torch.empty_like(w)
    moe_pack_bf16(E, N, K, w, out, stream)
    out._moe_layout = "packed"
    return out


def moe_pack_mxfp4(E, N, K, codes, scales, codes_out, scales_out, stream=None) -> None:
    """Repack OCP row-major MXFP4 matrices into the layout moe_forward reads."""
    _check(load().moe_pack_mxfp4(E, N, K, _ptr(codes), _ptr(scales), _ptr(codes_out),
                                 _ptr(scales_out), _stream(stream)))


def pack_mxfp4(codes, scales, stream=None):
    """Packed copies of codes [E, N, K/2] and scales [E, N, K/32] (uint8 device tensors)."""
    import torch
    E, N, K2 = codes.shape
    out_c = torch.empty_like(codes)
    out_s = torch.empty_like(scales)
    moe_pack_mxfp4(E, N, 2 * K2, codes, scales, out_c, out_s, stream)
    out_c._moe_layout = out_s._moe_layout = "packed"
    return out_c, out_s


STAGES = ("router", "permute", "gate_up", "down", "combine")


def moe_stage_timing_enable(on: bool) -> None:
    _check(load().moe_stage_timing_enable(1 if on else 0))


def moe_stage_timing_read():
    """(milliseconds summed per stage as a dict, number of timed calls)."""
    ms = (ctypes.c_float * len(STAGES))()
    n = ctypes.c_int(0)
    _check(load().moe_stage_timing_read(ms, len(STAGES), ctypes.byref(n)))
    return dict(zip(STAGES, [float(v) for v in ms])), n.value


def moe_probe_read(buf, stream=None) -> None:
    """Stream-read the device tensor `buf` (measurement aid, see moe.h)."""
    n = buf.numel() * buf.element_size()
    _check(load().moe_probe_read(_ptr(buf), n - n % 16, _stream(stream)))


def moe_probe_mfma(waves: int, iters: int, stream=None) -> None:
    """bf16 MFMA chains on every wave (measurement aid, see moe.h)."""
    _check(load().moe_probe_mfma(waves, iters, None, _stream(stream)))


def moe_probe_gather(pool, chunk_bytes: int, order, wgs: int, stream=None) -> None:
    """Read the chunks of `pool` listed in the int32 device tensor `order`
    (measurement aid, see moe.h)."""
    n = pool.numel() * pool.element_size()
    _check(load().moe_probe_gather(_ptr(pool), n, chunk_bytes, _ptr(order), order.numel(), wgs,
                                   _stream(stream)))


def moe_probe_mxfp4(codes, scales, out, stream=None) -> None:
    """Decode and sum the MXFP4 blocks of `codes` / `scales` (row-major OCP
    form); out (float32 device tensor) receives one sum per workgroup
    (measurement aid, see moe.h)."""
    nblk = scales.numel()
    assert codes.numel() * codes.element_size() >= 16 * nblk
    _check(load().moe_probe_mxfp4(_ptr(codes), _ptr(scales), nblk, out.numel(), _ptr(out),
                                  _stream(stream)))


def moe_strerror(code: int) -> str:
    return load().moe_strerror(code).decode()


def moe_last_error() -> str:
    return load().moe_last_error().decode()
