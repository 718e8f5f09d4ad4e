"""Pins of the CPU oracle against things other than itself.

* brute force: a dense numpy evaluation of every expert for every token,
  masked by the routing, with the softmax taken over all E experts first and
  renormalised over the selected ones (the literal reading of "renormalised
  softmax weights"), on tiny shapes;
* textbook special cases: E = k = 1 is a plain SwiGLU MLP (torch CPU);
* invariants: weights sum to one, k distinct in-range indices, bias shift
  invariance, expert relabelling, linearity in the down projection, x = 0;
* the storage formats against torch's bf16 and the OCP MX v1.0 tables;
* the numbers the pages print (tests/golden/pages.json).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


E2M1 = np.array(_gold("e2m1_ocp.json")["values"], dtype=np.float64)


# ---- independent decoders (numpy / torch, not the oracle's) --------------------

def dec(a, enc, scales=None):
    if enc == "f32":
        return np.asarray(a, np.float64)
    if enc == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    lo = a & 0xF
    hi = a >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(*a.shape[:-1], a.shape[-1] * 2)
    vals = E2M1[codes]
    s = np.exp2(scales.astype(np.float64) - 127.0)
    return vals * np.repeat(s, 32, axis=-1)


def brute_force(L: oracle.Layer, x):
    X = dec(x, L.act)
    Wr = dec(L.router_w, L.act)
    logits = X @ Wr.T
    if L.router_bias is not None:
        logits = logits + L.router_bias.astype(np.float64)[None, :]
    E, k = L.E, L.top_k
    p = np.exp(logits - logits.max(1, keepdims=True))
    p = p / p.sum(1, keepdims=True)
    ids = np.broadcast_to(np.arange(E), logits.shape)
    order = np.lexsort((ids, -logits), axis=-1)
    sel = order[:, :k]
    psel = np.take_along_axis(p, sel, 1)
    w = psel / psel.sum(1, keepdims=True)
    Wg = dec(L.w_gate, L.w, L.s_gate)
    Wu = dec(L.w_up, L.w, L.s_up)
    Wd = dec(L.w_down, L.w, L.s_down)
    G = np.einsum("th,eih->tei", X, Wg)
    U = np.einsum("th,eih->tei", X, Wu)
    A = G / (1.0 + np.exp(-G)) * U
    O = np.einsum("tei,ehi->teh", A, Wd)
    M = np.zeros((X.shape[0], E))
    np.put_along_axis(M, sel, w, 1)
    y = np.einsum("te,teh->th", M, O)
    if L.I_shared:
        Sg, Su, Sd = dec(L.sh_gate, L.act), dec(L.sh_up, L.act), dec(L.sh_down, L.act)
        g = X @ Sg.T
        y = y + (g / (1.0 + np.exp(-g)) * (X @ Su.T)) @ Sd.T
    return y, sel.astype(np.int32), w


def host_layer(c, device="cpu", wset=0) -> oracle.Layer:
    lay = mi.make_layer(c, device, wset)
    h = mi.to_host
    return oracle.Layer(H=c["H"], E=c["E"], top_k=c["top_k"], I=c["I"], act=c["act"], w=c["w"],
                        router_w=lay.router_w, router_bias=lay.router_bias,
                        w_gate=h(lay.w_gate), w_up=h(lay.w_up), w_down=h(lay.w_down),
                        s_gate=h(lay.s_gate), s_up=h(lay.s_up), s_down=h(lay.s_down),
                        I_shared=c["I_shared"], sh_gate=h(lay.sh_gate), sh_up=h(lay.sh_up),
                        sh_down=h(lay.sh_down))


def margin_x(c, L):
    return mi.make_x(c, reject=lambda x, rows: oracle.topk_margin(L, x, rows) < mi.MARGIN)


TINY = dict(T=24, H=64, E=6, top_k=2, I=32, I_shared=0, act="f32", w="f32", bias=None,
            layer="L0", seed=11)


@pytest.mark.parametrize("variant", ["f32", "bf16", "bias", "shared", "mxfp4", "k3"])
def test_forward_matches_brute_force(variant):
    c = dict(TINY)
    if variant == "bf16":
        c.update(act="bf16", w="bf16")
    elif variant == "bias":
        c.update(bias="uniform")
    elif variant == "shared":
        c.update(act="bf16", w="bf16", I_shared=48, bias="zipf1.1")
    elif variant == "mxfp4":
        c.update(act="bf16", w="mxfp4")
    elif variant == "k3":
        c.update(top_k=3, E=5)
    L = host_layer(c)
    x = margin_x(c, L)
    y, idx, w = oracle.forward(L, x)
    yb, idxb, wb = brute_force(L, x)
    assert np.array_equal(idx, idxb)
    np.testing.assert_allclose(w, wb, rtol=0, atol=1e-14)
    scale = np.abs(yb).max()
    assert scale > 0
    assert np.abs(y - yb).max() <= 1e-12 * scale
    # route() agrees with forward()
    idx2, w2, logits = oracle.route(L, x)
    assert np.array_equal(idx2, idx) and np.array_equal(w2, w)
    # token subsets give the same rows
    sub = np.array([5, 0, 17, 5], np.int32)
    ys, idxs, _ = oracle.forward(L, x, sub)
    assert np.array_equal(ys, y[sub]) and np.array_equal(idxs, idx[sub])


@pytest.mark.parametrize("shared", [False, True])
def test_single_expert_is_swiglu_mlp(shared):
    c = dict(TINY, E=1, top_k=1, I_shared=40 if shared else 0)
    L = host_layer(c)
    x = mi.make_x(c)
    y, idx, w = oracle.forward(L, x)
    assert (idx == 0).all() and (w == 1.0).all()
    F = torch.nn.functional
    X = torch.from_numpy(x.astype(np.float64))
    mlp = lambda g, u, d: F.silu(X @ torch.from_numpy(g.astype(np.float64)).T) * (
        X @ torch.from_numpy(u.astype(np.float64)).T) @ torch.from_numpy(d.astype(np.float64)).T
    ref = mlp(L.w_gate[0], L.w_up[0], L.w_down[0])
    if shared:
        ref = ref + mlp(L.sh_gate, L.sh_up, L.sh_down)
    ref = ref.numpy()
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()
    # the SiLU sits on the gate branch: swapping gate and up changes the answer
    swapped = mlp(L.w_up[0], L.w_gate[0], L.w_down[0]).numpy()
    if shared:
        swapped = swapped + mlp(L.sh_gate, L.sh_up, L.sh_down).numpy()
    assert np.abs(y - swapped).max() > 1e-3 * np.abs(ref).max()


def test_top1_weight_is_exactly_one():
    c = dict(TINY, top_k=1)
    L = host_layer(c)
    idx, w, logits = oracle.route(L, mi.make_x(c))
    assert (w == 1.0).all()
    assert np.array_equal(idx[:, 0], np.argmax(logits, axis=1))


def test_route_invariants_c1_shape():
    c = mi.cfg("c1", T=48)
    L = host_layer(dict(c, I=32))  # expert width does not enter routing
    x = mi.make_x(c)
    idx, w, logits = oracle.route(L, x)
    assert idx.shape == (48, 8)
    assert ((idx >= 0) & (idx < 256)).all()
    assert all(len(set(r)) == 8 for r in idx.tolist())
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-12)
    assert (np.diff(w, axis=1) <= 0).all()  # descending logits -> descending weights
    # the selected logits are the k largest
    srt = np.sort(logits, axis=1)[:, ::-1]
    np.testing.assert_array_equal(np.take_along_axis(logits, idx, 1), srt[:, :8])


def test_bias_shift_invariance():
    c = dict(TINY, bias="uniform", E=7, top_k=3)
    L = host_layer(c)
    # biases on a 2^-10 grid, so that adding 3 is exact in fp32
    L.router_bias = (np.round(L.router_bias * 1024) / 1024).astype(np.float32)
    x = mi.make_x(c)
    idx, w, _ = oracle.route(L, x)
    L.router_bias = (L.router_bias + np.float32(3.0)).astype(np.float32)
    idx2, w2, _ = oracle.route(L, x)
    assert np.array_equal(idx, idx2)
    np.testing.assert_allclose(w, w2, rtol=0, atol=1e-12)


def test_relabelling_experts():
    c = dict(TINY, E=6, top_k=3, act="bf16", w="bf16")
    L = host_layer(c)
    x = margin_x(c, L)
    y, idx, w = oracle.forward(L, x)
    perm = np.array([3, 5, 0, 1, 4, 2])  # new expert n is old expert perm[n]
    inv = np.argsort(perm)
    L2 = oracle.Layer(**{**L.__dict__})
    for name in ("router_w", "w_gate", "w_up", "w_down"):
        setattr(L2, name, np.ascontiguousarray(getattr(L, name)[perm]))
    y2, idx2, w2 = oracle.forward(L2, x)
    assert np.array_equal(idx2, inv[idx])
    assert np.array_equal(w2, w)
    assert np.array_equal(y2, y)


def test_down_projection_linearity_and_zero_input():
    c = dict(TINY)
    L = host_layer(c)
    x = mi.make_x(c)
    y, _, _ = oracle.forward(L, x)
    L2 = oracle.Layer(**{**L.__dict__})
    L2.w_down = (L.w_down * np.float32(2)).astype(np.float32)
    y2, _, _ = oracle.forward(L2, x)
    assert np.array_equal(y2, 2 * y)
    z = np.zeros_like(x)
    y0, idx0, w0 = oracle.forward(L, z)
    assert (y0 == 0).all()
    # all logits tie at zero: the lowest indices win, equal weights
    assert (idx0 == np.arange(c["top_k"])[None, :]).all()
    assert (w0 == 1.0 / c["top_k"]).all()


def test_bias_only_routing_and_margin():
    c = dict(TINY, E=6, top_k=2)
    L = host_layer(c)
    L.router_w = np.ascontiguousarray(np.repeat(L.router_w[:1], 6, axis=0))
    L.router_bias = np.array([0.0, 0.5, 0.25, 1.0, 0.5, -1.0], np.float32)
    x = mi.make_x(c)
    idx, w, _ = oracle.route(L, x)
    # order follows the bias: 3 (1.0), then the tie 1/4 (0.5) goes to 1
    assert (idx == np.array([3, 1])[None, :]).all()
    np.testing.assert_allclose(w[:, 0], 1 / (1 + math.exp(-0.5)), rtol=0, atol=1e-14)
    gap = oracle.topk_margin(L, x)
    assert (gap == 0.0).all()  # slots 2 and 3 (experts 1 and 4) tie
    L.router_bias = np.array([0.0, 0.5, 0.25, 1.0, 0.375, -1.0], np.float32)
    gap = oracle.topk_margin(L, x)
    np.testing.assert_allclose(gap, 0.125, rtol=0, atol=1e-12)


def test_permute_is_stable_grouping():
    rng = np.random.default_rng(7)
    for T, k, E in [(0, 2, 4), (1, 1, 1), (37, 3, 5), (300, 8, 256)]:
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32) \
            if T else np.zeros((0, k), np.int32)
        counts, offsets, row_src = oracle.permute(idx, E)
        flat = idx.reshape(-1)
        assert np.array_equal(counts, np.bincount(flat, minlength=E))
        assert offsets[0] == 0 and offsets[-1] == T * k
        assert np.array_equal(np.diff(offsets), counts)
        assert np.array_equal(row_src, np.argsort(flat, kind="stable"))


def test_bf16_decode_matches_torch():
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x7F7F, 0x0001, 0x4049, 0xC2F7, 0x3C23],
                    np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_to_f64(int(b)) for b in bits])
    assert np.array_equal(got, ref)
    # the generator's rounding agrees with torch's fp32 -> bf16 cast
    f = np.random.default_rng(3).standard_normal(4096).astype(np.float32)
    tb = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mi.bf16_bits(f), tb)


def test_e2m1_and_e8m0_tables():
    g = _gold("e2m1_ocp.json")
    for code, v in enumerate(g["values"]):
        got = oracle.e2m1_value(code)
        assert got == v and math.copysign(1, got) == math.copysign(1, v)
    for s, v in g["e8m0"]:
        assert oracle.e8m0_value(s) == v
    assert math.isnan(oracle.e8m0_value(255))


def test_mxfp4_decode_and_quantiser():
    w = torch.randn(16, 128, generator=torch.Generator().manual_seed(5)) * 0.02
    w[3, :32] = 0.0                       # an all-zero block
    w[4, 32:64] = torch.tensor([0.75, 1.25, 5.0, 2.5] * 8) * 2.0 ** -6  # ties
    codes, scales = mi.mxfp4_quantize(w)
    codes, scales = codes.numpy(), scales.numpy()
    d = oracle.decode(codes, "mxfp4", 16, 128, scales)
    assert np.array_equal(d, dec(codes, "mxfp4", scales))
    assert np.array_equal(oracle.decode(codes, "mxfp4", 16, 128, scales),
                          np.stack([[oracle.e2m1_value(int((codes[n, k // 2] >> (4 * (k % 2))) & 15))
                                     * oracle.e8m0_value(int(scales[n, k // 32]))
                                     for k in range(128)] for n in range(16)]))
    # quantisation error within half a grid step (step <= 2 * 2^e), saturation at 6 * 2^e
    e = scales.astype(np.float64) - 127
    step = np.repeat(np.exp2(e + 1), 32, axis=1)
    err = np.abs(d - w.double().numpy())
    sat = np.abs(w.double().numpy()) > 6 * np.repeat(np.exp2(e), 32, axis=1)
    assert (err[~sat] <= step[~sat] / 2 + 1e-18).all()
    assert (d[3, :32] == 0).all()
    # ties round to the even code (scale 2^-6): 0.75 -> 1, 1.25 -> 1, 5 -> 4, 2.5 -> 2
    assert scales[4, 1] == 127 - 6
    assert np.array_equal(d[4, 32:64] / 2.0 ** -6, np.array([1.0, 1.0, 4.0, 2.0] * 8))


def test_mxfp4_bytes_match_page():
    g = _gold("pages.json")["mxfp4_chunk_bytes"]
    N, K = g["N"], g["K"]
    codes, scales = mi.mxfp4_quantize(torch.zeros(1, N, K))
    nbytes = codes.numel() + scales.numel()
    assert nbytes == g["bytes"] == N * K * 17 // 32
    assert round(3 * nbytes / 2 ** 20, 1) == g["unit_mib"]


def expected_unique(E, k, Q):
    """Expected distinct experts touched by Q tokens choosing k of E each."""
    return E * (1 - (1 - k / E) ** Q)


def test_unique_expert_formula_matches_page():
    g = _gold("pages.json")
    u = g["unique_experts"]
    for Q, val in u["rows"]:
        assert round(expected_unique(u["E"], u["k"], Q), 1) == pytest.approx(val, abs=0.05 if val < 256 else 0.5)
    t = g["tokens_per_expert"]
    for Q, val in t["rows"]:
        assert Q * t["k"] / t["E"] == pytest.approx(val, abs=0.05)
    q = g["quantum_inverse"]
    assert q["target"] * q["E"] / q["k"] == q["Q"]


def test_router_touches_expected_experts_c1():
    c = mi.cfg("c1")
    L = host_layer(dict(c, I=32))
    idx, _, _ = oracle.route(L, mi.make_x(c))
    assert abs(len(np.unique(idx)) - expected_unique(256, 8, 128)) <= 8


def test_margin_filter_accepts_only_wide_gaps():
    c = dict(TINY, act="bf16", w="bf16")
    L = host_layer(c)
    x = margin_x(c, L)
    assert (oracle.topk_margin(L, x) >= mi.MARGIN).all()
    x0 = mi.make_x(c)
    changed = np.any(x0 != x, axis=1)
    gap0 = oracle.topk_margin(L, x0)
    assert np.array_equal(changed, gap0 < mi.MARGIN)


def test_zipf_bias_skews_loads():
    c = mi.cfg("c2", T=512)
    L = host_layer(dict(c, I=32))
    idx, _, _ = oracle.route(L, mi.make_x(c))
    counts = np.bincount(idx.reshape(-1), minlength=256)
    assert counts.max() > 0.9 * 512          # one expert takes nearly every token
    assert (counts > 0).sum() < 200          # many experts get none


def test_oracle_rejects_bad_arguments():
    c = dict(TINY)
    L = host_layer(c)
    x = mi.make_x(c)
    L.top_k = 7  # > E
    with pytest.raises(ValueError):
        oracle.route(L, x)
