"""Shared set-up of the GPU parity tests: inputs from ``moe_inputs``, the GPU
layer through the C-ABI binding, and the oracle on host copies of the same
inputs."""
from __future__ import annotations

import numpy as np
import torch

import moe_inputs as mi
import oracle
import routed_expert_ffn_moe_amd as moe

TOL = {"f32": 1e-4, "bf16": 2e-2, "mxfp4": 5e-2}  # max|y - y_ref| / max|y_ref|
# Self-imposed bars, tighter than the stated tolerances: a few times the
# errors the arithmetic gives (fp32 accumulation over K <= 256 for f32; h,
# staging rows and y rounded to bf16 once each for bf16; the same plus the
# hi/lo MXFP8 split of the activations, ~2^-8 relative, for MXFP4).
TIGHT = {"f32": 1e-5, "bf16": 1e-2, "mxfp4": 1e-2}
W_TOL = 1e-5                                     # routing weights, absolute


def oracle_layer(c, lay, experts=None) -> oracle.Layer:
    """Host view of the layer for the oracle.  With `experts`, only those
    experts' weights are copied (the rest of the host arrays stay untouched,
    unallocated pages)."""
    def host(t, sub=None):
        if t is None:
            return None
        if experts is None or sub is None:
            return mi.to_host(t)
        shape = tuple(t.shape)
        dt = np.uint16 if t.dtype == torch.bfloat16 else mi.to_host(t[:1]).dtype
        out = np.empty(shape, dt)
        for e in experts:
            out[e] = mi.to_host(t[e])
        return out

    return oracle.Layer(H=c["H"], E=c["E"], top_k=c["top_k"], I=c["I"], act=c["act"], w=c["w"],
                        router_w=lay.router_w, router_bias=lay.router_bias,
                        w_gate=host(lay.w_gate, 1), w_up=host(lay.w_up, 1),
                        w_down=host(lay.w_down, 1), s_gate=host(lay.s_gate, 1),
                        s_up=host(lay.s_up, 1), s_down=host(lay.s_down, 1),
                        I_shared=c["I_shared"], sh_gate=host(lay.sh_gate),
                        sh_up=host(lay.sh_up), sh_down=host(lay.sh_down))


def router_only_layer(c, lay) -> oracle.Layer:
    """Enough of the layer for routing (the margin filter, route())."""
    z = np.zeros((1,), np.uint16)
    return oracle.Layer(H=c["H"], E=c["E"], top_k=c["top_k"], I=c["I"], act=c["act"], w=c["w"],
                        router_w=lay.router_w, router_bias=lay.router_bias,
                        w_gate=z, w_up=z, w_down=z)


def margin_x(c, lay):
    L = router_only_layer(c, lay)
    return mi.make_x(c, reject=lambda x, rows: oracle.topk_margin(L, x, rows) < mi.MARGIN)


def act_torch(a: np.ndarray, act: str, dev):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if act == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(dev)


class GpuLayer:
    """Device tensors and the C-ABI weight struct of one layer."""

    def __init__(self, c, lay, dev="cuda"):
        self.c, self.lay, self.dev = c, lay, dev
        self.router_w = act_torch(lay.router_w, c["act"], dev)
        self.router_bias = None if lay.router_bias is None else torch.from_numpy(lay.router_bias).to(dev)
        wg, wu, wd = lay.w_gate, lay.w_up, lay.w_down
        sg, su, sd = lay.s_gate, lay.s_up, lay.s_down
        shg, shu, shd = lay.sh_gate, lay.sh_up, lay.sh_down
        # the layouts the kernels read
        if c["w"] == "mxfp4":
            (wg, sg), (wu, su), (wd, sd) = (moe.pack_mxfp4(wg, sg), moe.pack_mxfp4(wu, su),
                                            moe.pack_mxfp4(wd, sd))
        elif c["w"] == "bf16":
            wg, wu, wd = moe.pack_bf16(wg), moe.pack_bf16(wu), moe.pack_bf16(wd)
        if c["act"] == "bf16" and shg is not None:
            shg, shu, shd = moe.pack_bf16(shg), moe.pack_bf16(shu), moe.pack_bf16(shd)
        self.weights = moe.make_weights(self.router_w, wg, wu, wd,
                                        router_bias=self.router_bias, s_gate=sg,
                                        s_up=su, s_down=sd, sh_gate=shg,
                                        sh_up=shu, sh_down=shd)

    def shape(self, T, chunk_T=0):
        c = self.c
        return moe.make_shape(T, c["H"], c["E"], c["top_k"], c["I"], c["I_shared"], chunk_T,
                              c["act"], c["w"])

    def forward(self, x_dev, chunk_T=0, poison=False, ws=None):
        c = self.c
        T = x_dev.shape[0]
        shape = self.shape(T, chunk_T)
        nbytes = moe.moe_workspace_bytes(shape)
        if ws is None:
            ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.dev)
        y = torch.empty_like(x_dev)
        idx = torch.empty((T, c["top_k"]), dtype=torch.int32, device=self.dev)
        w = torch.empty((T, c["top_k"]), dtype=torch.float32, device=self.dev)
        if poison:  # NaN everywhere the layer writes or stages
            ws.fill_(0xFF)
            y.view(torch.uint8).fill_(0xFF)
            w.fill_(float("nan"))
            idx.fill_(-1)
        moe.moe_forward(shape, self.weights, x_dev, y, idx, w, ws)
        torch.cuda.synchronize()
        return y, idx, w

    def route(self, x_dev):
        c = self.c
        T = x_dev.shape[0]
        shape = self.shape(T)
        ws = torch.empty(max(moe.moe_workspace_bytes(shape), 256), dtype=torch.uint8, device=self.dev)
        idx = torch.empty((T, c["top_k"]), dtype=torch.int32, device=self.dev)
        w = torch.empty((T, c["top_k"]), dtype=torch.float32, device=self.dev)
        counts = torch.empty(c["E"], dtype=torch.int32, device=self.dev)
        offsets = torch.empty(c["E"] + 1, dtype=torch.int32, device=self.dev)
        row_src = torch.empty(max(T * c["top_k"], 1), dtype=torch.int32, device=self.dev)
        moe.moe_route(shape, self.weights, x_dev, idx, w, counts, offsets, row_src, ws)
        torch.cuda.synchronize()
        return idx, w, counts, offsets, row_src[: T * c["top_k"]]


def y_host(y: torch.Tensor, act: str) -> np.ndarray:
    if act == "bf16":
        return y.float().cpu().numpy().astype(np.float64)
    return y.cpu().numpy().astype(np.float64)


def rel_err(y, y_ref) -> float:
    scale = np.abs(y_ref).max()
    return float(np.abs(y - y_ref).max() / scale) if scale > 0 else float(np.abs(y).max())
