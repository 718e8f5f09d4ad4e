"""Host logic of bench.py (no GPU): the algorithmic bytes and flops of a
stage, the roofline verdict, the reading of committed counter records, and
the one-GPU refusal."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import moe_inputs as mi  # noqa: E402


def _counts(E, touched):
    c = np.zeros(E, np.int64)
    c[:touched] = 1
    return c


def test_gate_up_bytes_of_the_prefill_layer():
    """T=2048, H=2048, I=768, top-8 bf16 with 102 experts touched: the
    weights of 102 experts (2 x 768 x 2048 bf16 each, 641,728,512 bytes) and
    x once (8,388,608); the h rows (16,384 x 768 bf16) are the
    implementation's own traffic, reported apart."""
    w = bench.stage_work(mi.cfg("c2"), _counts(256, 102))
    assert w["_Es"] == 102
    assert w["gate_up"][0] == 641_728_512 + 8_388_608
    assert w["gate_up"][1] == 4.0 * 2048 * 8 * 2048 * 768  # 2 GEMMs x 2 flops per MAC
    # down: 102 experts' 2048 x 768 weights; y is the combine's
    assert w["down"][0] == 102 * 2048 * 768 * 2
    assert w["combine"][0] == 2048 * 2048 * 2
    assert w["_overhead"]["h"] == 2 * 16_384 * 768 * 2
    assert w["_overhead"]["staging"] == 2 * 16_384 * 2048 * 2


def test_layer_bytes_are_the_papers_sum():
    """The stages add up to Es*3*H*I*b_w + E*H*b_r + 3*H*I_s*b_w + T*H*(b_x +
    b_y) + 8*T*k: hand count for the wide layer with a shared expert."""
    c = mi.cfg("c3")
    w = bench.stage_work(c, _counts(384, 384))
    T, H, E, k, I, Is = 8192, 4096, 384, 6, 2048, 2048
    want = 384 * 3 * H * I * 2 + E * H * 2 + E * 4 + 3 * H * Is * 2 + T * H * 4 + 8 * T * k
    assert w["_layer"][0] == want
    # the stages' own figures differ only by x, which router and gate+up both read
    got = sum(v[0] for kk, v in w.items() if not kk.startswith("_"))
    assert got == want + T * H * 2
    r = bench.layer_roofline(w, 5.0, "bf16")
    assert r["roofline_us"] == pytest.approx(want / 8e12 * 1e6, rel=1e-4)


def test_mxfp4_weight_bytes_include_the_scales():
    """MXFP4: 16 code bytes and one scale byte per 32 weights (17/32 byte);
    the decode row touches 8 experts: 13,369,344 weight bytes; with the
    fused down+combine kernel y is written by the down stage."""
    w = bench.stage_work(mi.cfg("c4_t1"), _counts(256, 8), fused_down_combine=True)
    assert w["gate_up"][0] == 13_369_344 + 2048 * 2
    assert w["down"][0] == 6_684_672 + 2048 * 2
    assert w["combine"][0] == 0


def test_roofline_picks_the_binding_resource():
    c = mi.cfg("c2")
    w = bench.stage_work(c, _counts(256, 102))
    r = bench.roofline(w, "gate_up", 0.17872, "bf16")  # 178.72 us
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(650_117_120 / 178.72e-6 / 1e9, rel=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0, abs=1e-4)
    assert bench.mfma_frac(w, "gate_up", 0.17872, "bf16") == pytest.approx(
        103079215104.0 / 178.72e-6 / 2.5e15, abs=1e-4)
    # a stage whose matrix time exceeds its memory time is reported on MFMA
    m = bench.roofline({"x": (1.0e6, 1.0e13)}, "x", 10.0, "bf16")
    assert m["bound"] == "mfma" and m["unit"] == "TFLOP/s"
    assert m["achieved"] == pytest.approx(1000.0) and m["frac"] == pytest.approx(0.4)


def test_weight_sets_exceed_the_infinity_cache():
    """Decode shapes rotate weight sets until the touched weights of the
    rotation exceed twice the 256 MB infinity cache; prefill layers use one."""
    for name in ("c4_t1", "c4_t6"):
        c = mi.cfg(name)
        n = bench.weight_sets(c)
        per = min(c["T"] * c["top_k"], c["E"]) * 3 * c["H"] * c["I"] * 17 / 32
        assert 1 < n <= 16 and (n * per > 2 * bench.MALL_BYTES or n == 16)
    assert bench.weight_sets(mi.cfg("c2")) == 1
    assert bench.weight_sets(mi.cfg("c3")) == 1


def test_weight_sets_follow_the_touched_experts():
    """With the experts a call actually touches, a skewed router that keeps
    to a few experts gets the rotation its own bytes need: 40 MXFP4 experts
    of H=2048, I=768 are 100 MB per call, so six sets pass 512 MB."""
    c = mi.cfg("c4_p2048", T=16)
    per = 3 * c["H"] * c["I"] * 17 / 32
    assert bench.weight_sets(c) == 2           # 128 distinct experts assumed
    n = bench.weight_sets(c, touched=40)
    assert n == 6 and n * 40 * per > 2 * bench.MALL_BYTES
    assert bench.weight_sets(c, touched=1) == 16
    assert bench.weight_sets(mi.cfg("c2"), touched=200) == 1


def test_traffic_records_only_for_the_current_sources(tmp_path, monkeypatch):
    sha = bench.kernel_sources_sha1()
    (tmp_path / "hbm_traffic_counters.md").write_text(
        "# summary\n"
        '<!-- traffic {"workload": "c2", "stage": "gate_up", "bytes": 123, "sources_sha1": "%s"} -->\n'
        '<!-- traffic {"workload": "c2", "stage": "down", "bytes": 456, "sources_sha1": "0000"} -->\n'
        % sha)
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_traffic("c2", "gate_up") == 123
    assert bench.measured_traffic("c2", "down") is None  # taken on other kernel sources
    assert bench.measured_traffic("c1", "gate_up") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_clock_listing_parse():
    """sclk / mclk from the `rocm-smi --showclocks` listing format (levels
    numbered or 'S' for the sleep state), and None where a clock is absent."""
    line = ("GPU[0]\t\t: mclk clock level: 0: (2000Mhz) "
            "GPU[0]\t\t: sclk clock level: 1: (2225Mhz) ")
    assert bench.parse_clocks(line) == (2225, 2000)
    assert bench.parse_clocks("GPU[0] : sclk clock level: S: (102Mhz)") == (102, None)
    assert bench.parse_clocks("no clocks here") == (None, None)


def test_per_call_quantiles():
    q = bench.quantiles([float(v) for v in range(100, 0, -1)])  # 1..100 in any order
    assert q == {"calls": 100, "median": 51.0, "p10": 11.0, "p90": 90.0}
    assert bench.quantiles([7.0]) == {"calls": 1, "median": 7.0, "p10": 7.0, "p90": 7.0}


def test_source_digest_ignores_comments_and_layout():
    """The digest that ties counter records to the kernels covers code only:
    comments and whitespace leave it unchanged, string literals and code do
    not."""
    a = 'int f(int x) { return x + 1; } // one\n/* two\n */ const char *s = "// kept";'
    b = 'int f(int x)\n{\n    return x + 1;  /* other words */\n}\nconst char *s = "// kept";'
    assert bench.source_code_text(a) == bench.source_code_text(b)
    assert bench.source_code_text(a) != bench.source_code_text(a.replace("x + 1", "x + 2"))
    assert bench.source_code_text(a) != bench.source_code_text(a.replace('"// kept"', '"// gone"'))
    assert '"// kept"' in bench.source_code_text(a)
