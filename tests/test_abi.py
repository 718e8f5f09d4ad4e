"""The C ABI without a GPU: the library loads, exports every function that
include/moe.h declares, sizes workspaces, and rejects bad arguments with the
documented codes before touching any device (every case below carries at
least one argument error, so no kernel is ever launched, except the one
valid call, which runs only where the machine has no GPU driver at all)."""
import ctypes
import os
import re

import pytest

import routed_expert_ffn_moe_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = moe.load()
    names = _declared()
    assert {"moe_forward", "moe_route", "moe_workspace_bytes", "moe_strerror",
            "moe_last_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_strerror_codes():
    assert moe.moe_strerror(0) == "ok"
    for code in (moe.MOE_EINVAL, moe.MOE_EWORKSPACE, moe.MOE_EUNSUPPORTED, moe.MOE_EHIP):
        assert moe.moe_strerror(code) not in ("ok", "unknown error code")
    assert moe.moe_strerror(12345) == "unknown error code"


GOOD = dict(T=128, H=2048, E=256, top_k=8, I=768, I_shared=0, chunk_T=0, act="bf16", w="bf16")


def shape(**kw):
    d = dict(GOOD, **kw)
    return moe.make_shape(d["T"], d["H"], d["E"], d["top_k"], d["I"], d["I_shared"],
                          d["chunk_T"], d["act"], d["w"])


def test_workspace_bytes():
    n1 = moe.moe_workspace_bytes(shape())
    assert n1 > 0
    # chunking bounds the workspace by the pass size
    assert moe.moe_workspace_bytes(shape(T=4096, chunk_T=128)) == n1
    assert moe.moe_workspace_bytes(shape(T=4096)) > n1
    # h and staging rows: T*k bf16 rows of I and H, at least
    assert n1 >= 128 * 8 * (768 + 2048) * 2
    assert moe.moe_workspace_bytes(shape(T=0)) >= 0
    for bad in (dict(H=100), dict(E=0), dict(top_k=9, E=8), dict(I=0), dict(act="f32")):
        assert moe.moe_workspace_bytes(shape(**bad)) == 0, bad


class FakeW:
    """moe_weights_t with fake (never dereferenced) 256-aligned addresses."""

    def __init__(self, **over):
        base = 0x7F0000000000
        d = dict(router_w=base, w_gate=base + 0x1000, w_up=base + 0x2000, w_down=base + 0x3000,
                 layout=moe.MOE_LAYOUT_PACKED)
        d.update(over)
        self.c = moe.moe_weights_t(**d)


def call(sh, w=None, x=0x7F1000000000, y=0x7F2000000000, idx=0x7F3000000000, tw=None,
         ws=0x7F4000000000, ws_bytes=0):
    lib = moe.load()
    w = w or FakeW()
    return lib.moe_forward(ctypes.byref(sh) if sh is not None else None, ctypes.byref(w.c),
                           x, y, idx, tw, ws, ws_bytes, None)


@pytest.mark.parametrize("bad,code", [
    (dict(T=-1), moe.MOE_EINVAL),
    (dict(H=96), moe.MOE_EINVAL),
    (dict(E=0), moe.MOE_EINVAL),
    (dict(E=1024), moe.MOE_EINVAL),
    (dict(top_k=0), moe.MOE_EINVAL),
    (dict(top_k=17, E=64), moe.MOE_EINVAL),
    (dict(top_k=9, E=8), moe.MOE_EINVAL),
    (dict(I=100), moe.MOE_EINVAL),
    (dict(I_shared=-64), moe.MOE_EINVAL),
    (dict(I_shared=100), moe.MOE_EINVAL),
    (dict(chunk_T=-1), moe.MOE_EINVAL),
    (dict(act="f32", w="bf16"), moe.MOE_EUNSUPPORTED),
    (dict(act="f32", w="mxfp4"), moe.MOE_EUNSUPPORTED),
    (dict(w="mxfp4", H=2112), moe.MOE_EINVAL),
    (dict(w="mxfp4", I_shared=128), moe.MOE_EUNSUPPORTED),
])
def test_shape_errors(bad, code):
    assert call(shape(**bad)) == code
    assert moe.moe_last_error() != ""


def test_null_and_alignment_errors():
    assert moe.load().moe_forward(None, None, None, None, None, None, None, 0, None) == moe.MOE_EINVAL
    sh = shape()
    assert call(sh, w=FakeW(router_w=0)) == moe.MOE_EINVAL
    assert call(sh, w=FakeW(w_up=0x7F0000000008)) == moe.MOE_EINVAL
    assert call(sh, w=FakeW(router_bias=0x7F0000000002)) == moe.MOE_EINVAL
    assert call(sh, x=0) == moe.MOE_EINVAL
    assert call(sh, y=0x7F2000000004) == moe.MOE_EINVAL
    assert call(sh, idx=0) == moe.MOE_EINVAL
    assert call(sh, tw=0x7F5000000001) == moe.MOE_EINVAL
    assert call(sh, ws=0) == moe.MOE_EINVAL
    assert call(sh, ws=0x7F4000000010, ws_bytes=1 << 40) == moe.MOE_EINVAL  # not 256-aligned
    # MXFP4 without scales, shared expert without weights
    assert call(shape(w="mxfp4")) == moe.MOE_EINVAL
    assert call(shape(I_shared=768)) == moe.MOE_EINVAL


def test_weight_layout_must_be_declared():
    """bf16 and MXFP4 expert matrices are read in the packed layouts only: a
    struct that declares them row-major (the zero value) is refused, as is an
    f32 layer declared packed."""
    assert call(shape(), w=FakeW(layout=moe.MOE_LAYOUT_ROWMAJOR)) == moe.MOE_EINVAL
    assert "packed" in moe.moe_last_error()
    assert call(shape(), w=FakeW(layout=7)) == moe.MOE_EINVAL
    f32 = shape(act="f32", w="f32", H=256, I=128, E=8, top_k=2)
    assert call(f32, w=FakeW(layout=moe.MOE_LAYOUT_PACKED)) == moe.MOE_EINVAL
    assert "row-major" in moe.moe_last_error()
    # the binding declares PACKED only when every matrix came out of the packers
    import torch
    t = torch.zeros(4, 64, dtype=torch.bfloat16)
    assert moe.make_weights(t, t, t, t).c.layout == moe.MOE_LAYOUT_ROWMAJOR
    p = torch.zeros(4, 64, dtype=torch.bfloat16)
    p._moe_layout = "packed"
    assert moe.make_weights(t, p, p, p).c.layout == moe.MOE_LAYOUT_PACKED
    assert moe.make_weights(t, p, t, p).c.layout == moe.MOE_LAYOUT_ROWMAJOR


@pytest.mark.parametrize("kw", [
    dict(T=1 << 20, H=2048),                                 # T*H = 2^31
    dict(T=50000, H=4096, E=64, top_k=16, I=1024),            # rows*H > 2^31
    dict(T=300000, H=1024, E=1023, top_k=8, I=256),           # T*E*8 > 2^31
    dict(T=200000, H=1024, E=64, top_k=8, I=256, I_shared=2048),  # rows*I_shared
])
def test_pass_too_large_for_32bit_offsets(kw):
    """Passes whose token, staging or logit offsets would not fit 32 bits are
    refused before any launch; chunk_T brings the pass back into range."""
    sh = 0x7F0000100000
    w = FakeW(sh_gate=sh, sh_up=sh + 0x1000, sh_down=sh + 0x2000)
    assert call(shape(**kw), w=w, ws_bytes=1 << 50) == moe.MOE_EINVAL
    assert "32-bit" in moe.moe_last_error()
    assert moe.moe_workspace_bytes(shape(**kw)) == 0
    assert moe.moe_workspace_bytes(shape(**kw, chunk_T=1024)) > 0


def test_workspace_too_small():
    sh = shape()
    need = moe.moe_workspace_bytes(sh)
    assert call(sh, ws_bytes=need - 1) == moe.MOE_EWORKSPACE
    assert "workspace" in moe.moe_last_error()


def test_route_rejects_chunking():
    lib = moe.load()
    sh = shape(chunk_T=32)
    w = FakeW()
    rc = lib.moe_route(ctypes.byref(sh), ctypes.byref(w.c), 0x7F1000000000, 0x7F3000000000,
                       None, None, None, None, 0x7F4000000000, 1 << 40, None)
    assert rc == moe.MOE_EINVAL


def test_zero_tokens_returns_ok_without_touching_buffers():
    assert call(shape(T=0), x=0, y=0, idx=0, ws=0) == moe.MOE_OK


@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="a GPU driver is present: a valid call would launch on fake addresses")
def test_valid_call_without_a_device_fails_loudly():
    """Every argument is valid, so the call reaches the device check, which
    finds no HIP device: an error code and a message, never a CPU path."""
    sh = shape()
    nb = moe.moe_workspace_bytes(sh)
    lib = moe.load()
    assert call(sh, ws_bytes=nb) == moe.MOE_EHIP
    assert b"hipGetDevice" in lib.moe_last_error()


@pytest.mark.parametrize("E,N,K,ptrs", [
    (0, 32, 256, (16, 32, 48, 64)),           # no experts
    (2, 24, 256, (16, 32, 48, 64)),           # N not a multiple of 16
    (2, 32, 200, (16, 32, 48, 64)),           # K not a multiple of 128
    (2, 32, 256, (0, 32, 48, 64)),            # NULL codes
    (2, 32, 256, (16, 33, 48, 64)),           # misaligned scales
    (2, 32, 256, (1 << 20, 2 << 20, 1 << 20, 3 << 20)),  # codes_out aliases codes
])
def test_pack_mxfp4_rejects_bad_arguments(E, N, K, ptrs):
    lib = moe.load()
    rc = lib.moe_pack_mxfp4(E, N, K, *[ctypes.c_void_p(p) for p in ptrs], None)
    assert rc == moe.MOE_EINVAL
    assert "moe_pack_mxfp4" in moe.moe_last_error()


@pytest.mark.parametrize("E,N,K,ptrs", [
    (0, 64, 64, (16, 1 << 20)),          # no experts
    (2, 48, 64, (16, 1 << 20)),          # N not a multiple of 32
    (2, 64, 80, (16, 1 << 20)),          # K not a multiple of 32
    (2, 64, 64, (0, 1 << 20)),           # NULL input
    (2, 64, 64, (16, (1 << 20) + 8)),    # misaligned output
    (2, 64, 64, (1 << 20, (1 << 20) + 1024)),  # output overlaps the input
])
def test_pack_bf16_rejects_bad_arguments(E, N, K, ptrs):
    lib = moe.load()
    rc = lib.moe_pack_bf16(E, N, K, *[ctypes.c_void_p(p) for p in ptrs], None)
    assert rc == moe.MOE_EINVAL
    assert "moe_pack_bf16" in moe.moe_last_error()


def test_probe_argument_checks():
    """The measurement probes reject bad sizes before launching anything."""
    lib = moe.load()
    buf = ctypes.c_void_p(0x7F1000000000)
    assert lib.moe_probe_read(None, 1 << 20, None) == moe.MOE_EINVAL
    assert lib.moe_probe_read(buf, 0, None) == moe.MOE_EINVAL
    assert lib.moe_probe_read(buf, (1 << 20) + 8, None) == moe.MOE_EINVAL
    assert lib.moe_probe_mfma(0, 10, None, None) == moe.MOE_EINVAL
    assert lib.moe_probe_mfma(6, 10, None, None) == moe.MOE_EINVAL
    assert lib.moe_probe_mfma(8, 0, None, None) == moe.MOE_EINVAL
    assert "probe" in moe.moe_last_error()


def test_scattered_and_mxfp4_probe_argument_checks():
    """The scattered-read and MXFP4-stream probes check sizes, NULL and
    misaligned pointers and workgroup counts before launching anything."""
    lib = moe.load()
    P = ctypes.c_void_p
    pool, order, out = P(0x7F1000000000), P(0x7F2000000000), P(0x7F3000000000)
    mb = 1 << 20
    ok = (pool, 64 * mb, mb, order, 8, 256, None)
    bad = [
        (None,) + ok[1:],                       # no pool
        ok[:3] + (None,) + ok[4:],              # no order
        ok[:2] + (0,) + ok[3:],                 # empty chunk
        ok[:2] + (mb + 8,) + ok[3:],            # chunk not a multiple of 16
        (pool, mb // 2, mb) + ok[3:],           # chunk larger than the pool
        ok[:4] + (0,) + ok[5:],                 # no chunks
        ok[:5] + (0, None),                     # no workgroups
        ok[:5] + (65537, None),                 # too many workgroups
        (P(0x7F1000000008),) + ok[1:],          # misaligned pool
    ]
    for args in bad:
        assert lib.moe_probe_gather(*args) == moe.MOE_EINVAL, args
        assert "moe_probe_gather" in moe.moe_last_error()
    codes, scales = P(0x7F4000000000), P(0x7F5000000000)
    okm = (codes, scales, 1 << 16, 256, out, None)
    badm = [
        (None,) + okm[1:],
        (codes, None) + okm[2:],
        okm[:4] + (None, None),
        okm[:2] + (0,) + okm[3:],
        okm[:3] + (0,) + okm[4:],
        okm[:3] + (70000,) + okm[4:],
        (P(0x7F4000000004),) + okm[1:],
    ]
    for args in badm:
        assert lib.moe_probe_mxfp4(*args) == moe.MOE_EINVAL, args
        assert "moe_probe_mxfp4" in moe.moe_last_error()
