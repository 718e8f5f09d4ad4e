"""moe_forward_noalloc (the entry point that allocates nothing: its scratch
is the library's static device array) against moe_forward on the same
inputs: identical routing and y, on two calls in a row, the second with a
smaller input (the scratch then holds the first call's leftovers), for the
bf16 prefill layer and the MXFP4 layer (decode rows and prefill chunks).  The size refusal runs
without a GPU."""
import ctypes

import numpy as np
import pytest

import moe_inputs as mi
import routed_expert_ffn_moe_amd as moe


def test_noalloc_refuses_passes_beyond_its_scratch():
    """T=2048 at H=2048, E=256, top-8, I=768 needs ~104 MiB of scratch: refused
    with MOE_EWORKSPACE before any device work; chunks of 1024 fit."""
    lib = moe.load()
    big = moe.make_shape(2048, 2048, 256, 8, 768, 0, 0, "bf16", "bf16")
    assert moe.moe_workspace_bytes(big) > moe.MOE_NOALLOC_SCRATCH_BYTES
    w = moe.moe_weights_t(router_w=0x7F0000000000, w_gate=0x7F0000001000,
                          w_up=0x7F0000002000, w_down=0x7F0000003000,
                          layout=moe.MOE_LAYOUT_PACKED)
    rc = lib.moe_forward_noalloc(ctypes.byref(big), ctypes.byref(w), 0x7F1000000000,
                                 0x7F2000000000, 0x7F3000000000, None, None)
    assert rc == moe.MOE_EWORKSPACE
    assert "static scratch" in moe.moe_last_error()
    ok = moe.make_shape(2048, 2048, 256, 8, 768, 0, 1024, "bf16", "bf16")
    assert moe.moe_workspace_bytes(ok) <= moe.MOE_NOALLOC_SCRATCH_BYTES
    # invalid shapes report the argument, as moe_forward does
    bad = moe.make_shape(16, 100, 256, 8, 768, 0, 0, "bf16", "bf16")
    assert lib.moe_forward_noalloc(ctypes.byref(bad), ctypes.byref(w), 0x7F1000000000,
                                   0x7F2000000000, 0x7F3000000000, None, None) == moe.MOE_EINVAL


@pytest.mark.gpu
@pytest.mark.parametrize("name,T1,T2", [("c1", 128, 40), ("c1", 600, 300), ("c4_t6", 6, 1),
                                        ("c4_t6", 600, 300)])
def test_noalloc_matches_forward_on_two_calls(name, T1, T2):
    """Short passes (T <= 128: the one-launch routing), long passes (T = 600
    and 300: the segmented router and the one-launch permutation over 5 and
    3 blocks), the MXFP4 decode rows, and MXFP4 prefill chunks (T = 600: the
    streaming kernels' 32-row tiles; T = 300: the MXFP4 tile kernels)."""
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import harness as hx
    lib = moe.load()
    c = mi.cfg(name)
    g = hx.GpuLayer(c, mi.make_layer(c, "cuda"))
    for T in (T1, T2):
        cc = dict(c, T=T, seed=7000 + T)
        x = hx.act_torch(hx.margin_x(cc, g.lay), c["act"], "cuda")
        y0, i0, w0 = g.forward(x)
        shape = g.shape(T)
        y = torch.full_like(x, float("nan"))
        idx = torch.full((T, c["top_k"]), -1, dtype=torch.int32, device="cuda")
        w = torch.full((T, c["top_k"]), float("nan"), dtype=torch.float32, device="cuda")
        st = torch.cuda.current_stream().cuda_stream
        rc = lib.moe_forward_noalloc(ctypes.byref(shape), ctypes.byref(g.weights.c),
                                     x.data_ptr(), y.data_ptr(), idx.data_ptr(), w.data_ptr(), st)
        assert rc == moe.MOE_OK, moe.moe_last_error()
        torch.cuda.synchronize()
        assert torch.equal(idx, i0) and torch.equal(w, w0), (name, T)
        assert torch.equal(y, y0), (name, T)
        # and against the oracle, as every other entry point is held
        import oracle
        xh = hx.margin_x(cc, g.lay)
        idx_r, _, _ = oracle.route(hx.router_only_layer(cc, g.lay), xh)
        assert np.array_equal(idx.cpu().numpy(), idx_r)
        experts = sorted(set(idx_r.reshape(-1).tolist()))
        y_ref, _, _ = oracle.forward(hx.oracle_layer(cc, g.lay, experts), xh)
        assert hx.rel_err(hx.y_host(y, c["act"]), y_ref) <= hx.TIGHT[c["w"]]
