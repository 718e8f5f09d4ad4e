"""Seeded synthetic inputs for the routed-expert MoE FFN layer.

This module only draws random tensors and encodes them into their storage
formats; it holds none of the layer's arithmetic.  Both the GPU library's
tests/benchmark and the CPU oracle take their inputs from here.

* Activations ``x`` and router weights come from numpy PCG64 streams keyed
  by ``SeedSequence([BASE, tag, ...])`` and are identical on every machine.
* Expert weights are large (up to 19.3 GB at the widest workload), so they
  are drawn with a seeded ``torch.Generator`` on the device that will hold
  them; their values depend on that device type.  Whatever consumes them on
  the host copies them from that device.
* bf16 values are the round-to-nearest-even of an fp32 draw.
* MXFP4 weights are fp32 draws quantised per 32-element block along K with
  the OCP MX v1.0 recipe: shared exponent floor(log2(amax)) - 2, elements
  rounded to nearest-even onto the E2M1 grid and saturated at +-6.
* Token rows can be redrawn until a caller-supplied predicate accepts them
  (used for the top-k margin filter; the predicate is the caller's, this
  module computes no logits).  Redraw ``a`` of row ``t`` uses its own stream
  ``SeedSequence([BASE, TAG_X, seed, t, a])``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, Optional

import numpy as np

BASE = 0x4D6F45  # fixed root of every stream
TAG_X, TAG_ROUTER, TAG_BIAS, TAG_GATE, TAG_UP, TAG_DOWN = 1, 2, 3, 4, 5, 6
TAG_SH_GATE, TAG_SH_UP, TAG_SH_DOWN, TAG_PERM = 7, 8, 9, 10
MAX_REDRAWS = 64

# The five workloads (C4 appears twice: the 6-row verify block and T=1).
# `layer` names the weight set; configurations naming the same layer share it.
CONFIGS: Dict[str, dict] = {
    "c0": dict(T=64, H=256, E=8, top_k=2, I=128, I_shared=0, act="f32", w="f32",
               bias=None, layer="L0", seed=0,
               desc="tiny fp32 layer: T=64 H=256 E=8 top-2 I=128"),
    "c1": dict(T=128, H=2048, E=256, top_k=8, I=768, I_shared=0, act="bf16", w="bf16",
               bias=None, layer="L1", seed=1,
               desc="small-chunk prefill: T=128 H=2048 E=256 top-8 I=768 bf16"),
    "c2": dict(T=2048, H=2048, E=256, top_k=8, I=768, I_shared=0, act="bf16", w="bf16",
               bias="zipf1.1", layer="L1", seed=2,
               desc="large-chunk prefill, Zipf(1.1) expert bias: T=2048 H=2048 E=256 top-8 I=768 bf16"),
    "c3": dict(T=8192, H=4096, E=384, top_k=6, I=2048, I_shared=2048, act="bf16", w="bf16",
               bias="uniform", layer="L3", seed=3,
               desc="wide layer + shared expert: T=8192 H=4096 E=384 top-6 I=2048 I_s=2048 bf16"),
    "c4_t6": dict(T=6, H=2048, E=256, top_k=8, I=768, I_shared=0, act="bf16", w="mxfp4",
                  bias=None, layer="L4", seed=4,
                  desc="verify block, MXFP4 experts: T=6 H=2048 E=256 top-8 I=768"),
    "c4_t1": dict(T=1, H=2048, E=256, top_k=8, I=768, I_shared=0, act="bf16", w="mxfp4",
                  bias=None, layer="L4", seed=5,
                  desc="decode row, MXFP4 experts: T=1 H=2048 E=256 top-8 I=768"),
    # the MXFP4 layer at a prefill chunk, skewed like the T=2048 bf16 chunk
    "c4_p2048": dict(T=2048, H=2048, E=256, top_k=8, I=768, I_shared=0, act="bf16",
                     w="mxfp4", bias="zipf1.1", layer="L4", seed=6,
                     desc="prefill chunk, MXFP4 experts, Zipf(1.1) expert bias: "
                          "T=2048 H=2048 E=256 top-8 I=768"),
}
LAYER_SEED = {"L0": 100, "L1": 101, "L3": 103, "L4": 104,
              # small layers of other shapes (the tests' sweep of kernel variants)
              "SA": 201, "SB": 202, "SC": 203, "SD": 204, "SE": 205, "SF": 206, "SG": 207,
              "SH": 208, "SI": 209, "SJ": 210, "SK": 211}
W_STD = 0.02      # std of router and expert weights
MARGIN = 1e-3     # minimum top-k logit gap of accepted token rows


def cfg(name: str, **override) -> dict:
    c = dict(CONFIGS[name])
    c.update(override)
    return c


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE, *key])))


# ---- storage encodings ------------------------------------------------------

def bf16_bits(f: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def encode_act(f: np.ndarray, act: str) -> np.ndarray:
    return bf16_bits(f) if act == "bf16" else np.ascontiguousarray(f, np.float32)


_E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def mxfp4_quantize(w):
    """OCP MX v1.0 MXFP4 encoding of a torch fp32 tensor [..., N, K] (K % 32 == 0).

    Returns (codes uint8 [..., N, K/2], scales uint8 [..., N, K/32]).
    """
    import torch
    *lead, N, K = w.shape
    assert K % 32 == 0
    blk = w.reshape(*lead, N, K // 32, 32)
    amax = blk.abs().amax(dim=-1)
    e = torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)))) - 2
    e = e.clamp(-127, 127)
    scale_code = torch.where(amax > 0, e + 127, torch.zeros_like(e)).to(torch.uint8)
    q = blk / torch.exp2(e)[..., None]
    a = q.abs().clamp(max=6.0)
    grid = torch.tensor(_E2M1_GRID, dtype=w.dtype, device=w.device)
    lo = (torch.searchsorted(grid, a.contiguous(), right=True) - 1).clamp(0, 7)
    hi = (lo + 1).clamp(max=7)
    dlo = a - grid[lo]
    dhi = grid[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0) & (hi != lo))
    mag = torch.where(pick_hi, hi, lo)
    sign = ((q < 0) & (mag > 0)).to(torch.int64)
    code = (mag | (sign << 3)).to(torch.uint8).reshape(*lead, N, K)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return packed.contiguous(), scale_code.contiguous()


# ---- layers -----------------------------------------------------------------

@dataclass
class LayerData:
    c: dict
    router_w: np.ndarray                    # host, act encoding [E, H]
    router_bias: Optional[np.ndarray]       # host float32 [E] or None
    w_gate: "object"                        # torch tensors on `device`
    w_up: "object"
    w_down: "object"
    s_gate: "object" = None
    s_up: "object" = None
    s_down: "object" = None
    sh_gate: "object" = None
    sh_up: "object" = None
    sh_down: "object" = None
    extra: dict = field(default_factory=dict)


def _torch_gen(device, *key):
    import torch
    seed = int(np.random.SeedSequence([BASE, *key]).generate_state(1, np.uint64)[0] >> 1)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _draw_matrices(device, E, N, K, key, std, enc):
    """E matrices [N, K] ~ N(0, std^2), encoded as `enc` (f32 | bf16 | mxfp4)."""
    import torch
    g = _torch_gen(device, *key)
    if enc == "mxfp4":
        codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device=device)
        scales = torch.empty((E, N, K // 32), dtype=torch.uint8, device=device)
    else:
        dt = torch.bfloat16 if enc == "bf16" else torch.float32
        out = torch.empty((E, N, K), dtype=dt, device=device)
    for e in range(E):
        w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32) * std
        if enc == "mxfp4":
            codes[e], scales[e] = mxfp4_quantize(w)
        else:
            out[e] = w.to(out.dtype)  # torch's fp32 -> bf16 cast rounds to nearest even
    return (codes, scales) if enc == "mxfp4" else (out, None)


def router_bias(c: dict) -> Optional[np.ndarray]:
    E, kind = c["E"], c["bias"]
    if kind is None:
        return None
    if kind.startswith("zipf"):
        s = float(kind[4:])
        rank = 1 + _rng(TAG_PERM, LAYER_SEED[c["layer"]]).permutation(E)
        return (-s * np.log(rank.astype(np.float64))).astype(np.float32)
    if kind == "uniform":
        return _rng(TAG_BIAS, LAYER_SEED[c["layer"]]).random(E, dtype=np.float32)
    raise ValueError(kind)


def make_layer(c: dict, device="cpu", wset: int = 0) -> LayerData:
    """Weights of configuration `c`'s layer; `wset` selects an independent copy."""
    ls = LAYER_SEED[c["layer"]]
    E, H, I, Is = c["E"], c["H"], c["I"], c["I_shared"]
    rw = _rng(TAG_ROUTER, ls, wset).standard_normal((E, H), dtype=np.float32) * np.float32(W_STD)
    lay = LayerData(c=c, router_w=encode_act(rw, c["act"]), router_bias=router_bias(c),
                    w_gate=None, w_up=None, w_down=None)
    lay.w_gate, lay.s_gate = _draw_matrices(device, E, I, H, (TAG_GATE, ls, wset), W_STD, c["w"])
    lay.w_up, lay.s_up = _draw_matrices(device, E, I, H, (TAG_UP, ls, wset), W_STD, c["w"])
    lay.w_down, lay.s_down = _draw_matrices(device, E, H, I, (TAG_DOWN, ls, wset), W_STD, c["w"])
    if Is:
        lay.sh_gate = _draw_matrices(device, 1, Is, H, (TAG_SH_GATE, ls, wset), W_STD, c["act"])[0][0]
        lay.sh_up = _draw_matrices(device, 1, Is, H, (TAG_SH_UP, ls, wset), W_STD, c["act"])[0][0]
        lay.sh_down = _draw_matrices(device, 1, H, Is, (TAG_SH_DOWN, ls, wset), W_STD, c["act"])[0][0]
    return lay


# ---- token rows ---------------------------------------------------------------

def make_x(c: dict, reject: Optional[Callable[[np.ndarray, np.ndarray], np.ndarray]] = None,
           seed: Optional[int] = None) -> np.ndarray:
    """Activations x [T, H] ~ N(0, 1) in the act encoding.

    `reject(x, rows)` returns a boolean mask over `rows` of rows to redraw;
    each redraw of row t uses its own stream.  Raises if a row is still
    rejected after MAX_REDRAWS attempts.
    """
    T, H = c["T"], c["H"]
    s = c["seed"] if seed is None else seed
    x = encode_act(_rng(TAG_X, s).standard_normal((T, H), dtype=np.float32), c["act"])
    if reject is None or T == 0:
        return x
    rows = np.arange(T, dtype=np.int64)
    for attempt in range(1, MAX_REDRAWS + 1):
        bad = rows[np.asarray(reject(x, rows), dtype=bool)]
        if bad.size == 0:
            return x
        for t in bad:
            f = _rng(TAG_X, s, int(t), attempt).standard_normal(H, dtype=np.float32)
            x[t] = encode_act(f, c["act"])
        rows = bad
    raise RuntimeError("token rows still rejected after %d redraws" % MAX_REDRAWS)


def to_host(t) -> np.ndarray:
    """Host numpy copy of a torch tensor in the storage convention (bf16 -> uint16)."""
    import torch
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().contiguous().cpu().numpy()
