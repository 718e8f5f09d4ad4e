#!/usr/bin/env python3
"""MoE-layer throughput of the gfx950 routed-expert FFN layer on one MI355X.

One step = one moe_forward over one chunk of synthetic tokens (router,
permutation, grouped gate+up with SwiGLU, grouped down with the routing-weight
scale, combine), inputs and weights already resident in HBM.  The default
workload is the large-chunk prefill layer: T=2048 tokens, H=2048, 256
experts top-8, I=768, bf16, Zipf(1.1) expert bias.  Also reported: the T=128
chunk of the same layer and the MXFP4 decode/verify shapes (T=6, T=1), per
stage timings from HIP events on the launch stream, the roofline of the
dominant kernel, and the CPU oracle timed on a bounded sample.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at chunk T=2048 (and T=128, T=6); % MFMA peak / HBM GB/s"
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "mxfp4": 10100.0, "f32": 157.3}
MALL_BYTES = 256 << 20


def stage_work(c, counts, fused_down_combine=False):
    """Algorithmic bytes and flops of each stage for one call: the operands
    the method itself must read and the outputs it must write, each once;
    expert weights only for the experts that received tokens (Es).  Over the
    whole layer the bytes add up to Es*3*H*I*b_w + E*H*b_r + 3*H*I_s*b_w +
    T*H*(b_x + b_y) + 8*T*k.  The intermediate h rows, the per-pair staging
    rows and the permutation's index arrays are the implementation's own
    traffic: `_overhead` gives their bytes (written once and read once),
    reported beside the algorithmic figure, never inside it.  With
    `fused_down_combine` (MXFP4 decode rows) y is written by the down stage."""
    T, H, E, k, I, Is = c["T"], c["H"], c["E"], c["top_k"], c["I"], c["I_shared"]
    a = 4 if c["act"] == "f32" else 2
    bw = {"f32": 4.0, "bf16": 2.0, "mxfp4": 17.0 / 32.0}[c["w"]]
    Es = int((counts > 0).sum())
    pairs = T * k
    rows = pairs + (T if Is else 0)
    y_bytes = T * H * a
    return {
        "router": (T * H * a + E * H * a + (E * 4 if c["bias"] else 0) + pairs * 8,
                   2.0 * T * H * E),
        "permute": (0.0, 0.0),
        "gate_up": (Es * 2 * I * H * bw + 2 * Is * H * a + T * H * a,
                    4.0 * pairs * H * I + 4.0 * T * H * Is),
        "down": (Es * H * I * bw + H * Is * a + (y_bytes if fused_down_combine else 0),
                 2.0 * pairs * H * I + 2.0 * T * H * Is),
        "combine": (0.0 if fused_down_combine else y_bytes, float(rows * H)),
        "_Es": Es,
        # the layer reads x once (router and gate+up each count it above)
        "_layer": (Es * 3 * H * I * bw + E * H * a + (E * 4 if c["bias"] else 0)
                   + 3 * H * Is * a + T * H * 2 * a + pairs * 8,
                   2.0 * T * H * E + 6.0 * pairs * H * I + 6.0 * T * H * Is),
        "_overhead": {"h": 2 * (pairs * I + T * Is) * a,
                      "staging": 0 if fused_down_combine else 2 * rows * H * a,
                      "permutation": pairs * 4 * 3},
    }


PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")


def source_code_text(src):
    """C/C++/HIP source text with its comments removed and its whitespace
    collapsed (string and character literals kept as they are)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
            out.append(" ")
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_sources_sha1():
    """Digest of the HIP sources' code (comments and whitespace left out):
    counter readings taken from other code no longer describe the kernels
    that run."""
    import hashlib
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "routed_expert_ffn_moe_amd", "csrc")
    h = hashlib.sha1()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(f.encode())
            with open(os.path.join(d, f), encoding="utf-8", errors="surrogateescape") as fh:
                h.update(source_code_text(fh.read()).encode("utf-8", "surrogateescape"))
    return h.hexdigest()


def measured_traffic(workload, stage):
    """HBM bytes per launch of `stage` on `workload` from the committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, each scaled by its
    reading for a plain copy), or None if there is none for the current
    kernel sources."""
    path = os.path.join(PROFILES, "hbm_traffic_counters.md")
    if not os.path.exists(path):
        return None
    sha = kernel_sources_sha1()
    for line in open(path):
        line = line.strip()
        if line.startswith("<!-- traffic ") and line.endswith("-->"):
            rec = json.loads(line[len("<!-- traffic "):-3])
            if rec.get("workload") == workload and rec.get("stage") == stage \
                    and rec.get("sources_sha1") == sha:
                return int(rec["bytes"])
    return None


def roofline(work, stage, ms, dtype):
    """The stage against the resource that bounds it: algorithmic bytes over
    8 TB/s or flops over the dense MFMA peak of its dtype, whichever takes
    longer at peak; `achieved` is that figure per second of the measured
    stage time."""
    byts, flops = work[stage]
    dur = ms / 1e3
    t_hbm = byts / (PEAK_HBM_GBS * 1e9)
    t_mma = flops / (PEAK_TFLOPS[dtype] * 1e12)
    common = {"traffic": None, "kernel": stage, "avg_us": round(ms * 1e3, 2),
              "alg_bytes": int(byts), "alg_flops": flops}
    if t_mma > t_hbm:
        ach = flops / dur / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_TFLOPS[dtype],
                "unit": "TFLOP/s", "frac": round(ach / PEAK_TFLOPS[dtype], 4), **common}
    ach = byts / dur / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), **common}


def mfma_frac(work, stage, ms, dtype):
    """Useful matrix flops of the stage per second against the dense peak of
    its dtype (padding rows not counted)."""
    return round(work[stage][1] / (ms / 1e3) / 1e12 / PEAK_TFLOPS[dtype], 4)


def layer_roofline(work, ms_step, dtype):
    """The whole layer call against its roofline: the layer's algorithmic
    bytes at 8 TB/s or its flops at the MFMA peak, whichever is longer."""
    byts, flops = work["_layer"]
    t_roof = max(byts / (PEAK_HBM_GBS * 1e9), flops / (PEAK_TFLOPS[dtype] * 1e12))
    return {"alg_bytes": int(byts), "alg_flops": flops, "roofline_us": round(t_roof * 1e6, 2),
            "measured_us": round(ms_step * 1e3, 2), "frac": round(t_roof / (ms_step / 1e3), 4)}


def weight_sets(c, touched=None):
    """Independent weight sets to rotate through so that consecutive calls
    find their expert weights in HBM, not in the 256 MB infinity cache: one
    when a call touches more than twice that, else enough sets (at most 16)
    to exceed it twice over.  `touched` is the number of experts one call
    routes to; without it every pair is taken to pick a distinct expert,
    which a skewed router bias makes far too many (Zipf(1.1) at T=16 reaches
    about a third of them)."""
    if touched is None:
        touched = min(c["top_k"] * c["T"], c["E"])
    per_call = touched * 3 * c["H"] * c["I"] * (17.0 / 32.0 if c["w"] == "mxfp4" else 2)
    return 1 if per_call > 2 * MALL_BYTES else int(min(16, 2 * MALL_BYTES // max(per_call, 1) + 1))


class Workload:
    def __init__(self, name, wsets=None, dev="cuda", keep_rowmajor=False, cfg=None):
        import torch

        import moe_inputs as mi
        import routed_expert_ffn_moe_amd as moe
        self.torch, self.moe = torch, moe
        self.name = name
        self.keep_rowmajor = keep_rowmajor
        self.c = dict(cfg) if cfg is not None else mi.cfg(name)
        c = self.c
        self.mi, self.dev = mi, dev
        x = mi.make_x(c)
        self.x_host = x
        t = torch.from_numpy(x)
        self.x = (t.view(torch.int16).view(torch.bfloat16) if c["act"] == "bf16" else t).to(dev)
        self.shape = moe.make_shape(c["T"], c["H"], c["E"], c["top_k"], c["I"], c["I_shared"],
                                    0, c["act"], c["w"])
        nb = moe.moe_workspace_bytes(self.shape)
        self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        self.y = torch.empty_like(self.x)
        self.idx = torch.empty((c["T"], c["top_k"]), dtype=torch.int32, device=dev)
        self.w = torch.empty((c["T"], c["top_k"]), dtype=torch.float32, device=dev)
        self.i = 0
        self.layers, self.weights, self._keep = [], [], []
        self._add_set(0)
        if wsets is None:
            # one routed call on the first set counts the experts a call touches
            self.step()
            self.i = 0
            wsets = weight_sets(c, int((self.counts() > 0).sum()))
        for s in range(1, wsets):
            self._add_set(s)

    def _add_set(self, s):
        """Draws weight set s, packs it and appends it to the rotation."""
        torch, moe, c = self.torch, self.moe, self.c
        lay = self.mi.make_layer(c, self.dev, s)
        self.layers.append(lay)
        dev = self.dev
        rw = torch.from_numpy(lay.router_w)
        rw = (rw.view(torch.int16).view(torch.bfloat16) if c["act"] == "bf16" else rw).to(dev)
        rb = None if lay.router_bias is None else torch.from_numpy(lay.router_bias).to(dev)
        self._keep += [rw, rb]
        wg, wu, wd = lay.w_gate, lay.w_up, lay.w_down
        sg, su, sd = lay.s_gate, lay.s_up, lay.s_down
        shg, shu, shd = lay.sh_gate, lay.sh_up, lay.sh_down
        # one-time repack into the layouts the kernels read (the row-major
        # copies go, so that the widest layer still fits twice over)
        if c["w"] == "mxfp4":
            (wg, sg), (wu, su), (wd, sd) = (moe.pack_mxfp4(wg, sg), moe.pack_mxfp4(wu, su),
                                            moe.pack_mxfp4(wd, sd))
        elif c["w"] == "bf16":
            wg, wu, wd = (self._packed(lay, "w_gate"), self._packed(lay, "w_up"),
                          self._packed(lay, "w_down"))
        if c["act"] == "bf16" and shg is not None:
            shg, shu, shd = (self._packed(lay, "sh_gate"), self._packed(lay, "sh_up"),
                             self._packed(lay, "sh_down"))
        self._keep += [wg, wu, wd, sg, su, sd, shg, shu, shd]
        self.weights.append(moe.make_weights(rw, wg, wu, wd, router_bias=rb, s_gate=sg,
                                             s_up=su, s_down=sd, sh_gate=shg,
                                             sh_up=shu, sh_down=shd))

    def step(self):
        wt = self.weights[self.i % len(self.weights)]
        self.i += 1
        self.moe.moe_forward(self.shape, wt, self.x, self.y, self.idx, self.w, self.ws)

    def warm(self, seconds=0.05):
        """Untimed bursts of 10 calls until `seconds` have passed: calls that
        start after the device has idled (input generation, another
        workload) run 10-20% slower for their first milliseconds."""
        t0 = time.perf_counter()
        while True:
            for _ in range(10):
                self.step()
            self.torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                return

    def time(self, steps, warmup):
        """Wall-clock seconds of exactly `steps` calls after `warmup` untimed
        ones, with a synchronisation on both sides, and the per-stage HIP-event
        times (ms per call) of a pass of the same calls made before them.
        Untimed warm-up bursts precede the stage pass, and the stage pass
        precedes the timed calls, so that both run at the clocks the layer
        sustains rather than in the slower first milliseconds after the
        device has idled."""
        torch, moe = self.torch, self.moe
        self.warm()
        moe.moe_stage_timing_enable(True)
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        ms, n = moe.moe_stage_timing_read()
        moe.moe_stage_timing_enable(False)
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall, {k: v / max(n, 1) for k, v in ms.items()}

    def per_call(self, steps):
        """Each call timed on its own with HIP events on the launch stream:
        median, p10 and p90 in microseconds."""
        torch = self.torch
        st = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            a.record(st)
            self.step()
            b.record(st)
        torch.cuda.synchronize()
        return quantiles([a.elapsed_time(b) * 1e3 for a, b in ev])

    def time_graph(self, steps, warmup):
        """Per-step time with the whole layer replayed from HIP graphs (one
        graph per weight set), for launch-bound decode shapes."""
        torch = self.torch
        s = torch.cuda.Stream()
        graphs = []
        with torch.cuda.stream(s):
            for _ in range(len(self.weights)):
                self.step()  # warm the kernels up outside capture
            torch.cuda.synchronize()
            for i in range(len(self.weights)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    self.moe.moe_forward(self.shape, self.weights[i], self.x, self.y, self.idx,
                                         self.w, self.ws)
                graphs.append(g)
        for i in range(warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def _packed(self, lay, name):
        """Packed copy of one bf16 matrix of `lay`; the row-major original is
        kept only for the primary workload (the CPU baseline reads it)."""
        w = getattr(lay, name)
        out = self.moe.pack_bf16(w)
        self.torch.cuda.synchronize()
        if not self.keep_rowmajor:
            setattr(lay, name, None)
        return out

    def counts(self):
        import numpy as np
        idx = self.idx.cpu().numpy()
        return np.bincount(idx.reshape(-1), minlength=self.c["E"])


def quantiles(us):
    """Median, p10 and p90 (nearest rank) of a list of microsecond figures."""
    v = sorted(us)
    q = lambda f: v[min(len(v) - 1, int(round(f * (len(v) - 1))))]
    return {"calls": len(v), "median": round(q(0.5), 2), "p10": round(q(0.1), 2),
            "p90": round(q(0.9), 2)}


def parse_clocks(text):
    """(sclk MHz, mclk MHz) from one `rocm-smi --showclocks` listing (None
    where a clock is not listed)."""
    import re
    out = {}
    for name in ("sclk", "mclk"):
        m = re.search(r"%s clock level:\s*\S+:?\s*\((\d+)\s*Mhz\)" % name, text, re.IGNORECASE)
        out[name] = int(m.group(1)) if m else None
    return out["sclk"], out["mclk"]


def clock_log(run, seconds=2.0, period=0.25):
    """Shader and memory clocks while `run(stop)` keeps the GPU busy for
    `seconds`: `rocm-smi --showclocks` sampled every `period` seconds from a
    child process; None where the tool is missing or lists no clocks."""
    import shutil
    import subprocess
    import threading
    tool = shutil.which("rocm-smi") or ("/opt/rocm/bin/rocm-smi"
                                        if os.path.exists("/opt/rocm/bin/rocm-smi") else None)
    if tool is None:
        return None
    samples, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                r = subprocess.run([tool, "--showclocks"], capture_output=True, text=True,
                                   timeout=5)
                samples.append(parse_clocks(r.stdout))
            except (OSError, subprocess.SubprocessError):
                pass
            stop.wait(period)

    th = threading.Thread(target=sample, daemon=True)
    t_end = time.perf_counter() + seconds
    th.start()
    try:
        run(lambda: time.perf_counter() >= t_end)
    finally:
        stop.set()
        th.join()
    # the first samples can fall before the load reaches the clocks
    busy = samples[2:] if len(samples) > 4 else samples

    def summary(vals):
        vals = sorted(v for v in vals if v is not None)
        if not vals:
            return None
        return {"min": vals[0], "median": vals[len(vals) // 2], "max": vals[-1],
                "samples": len(vals)}
    s_clk, m_clk = summary([a for a, _ in busy]), summary([b for _, b in busy])
    if s_clk is None and m_clk is None:
        return None
    return {"sclk_mhz": s_clk, "mclk_mhz": m_clk, "tool": "rocm-smi --showclocks",
            "window_s": seconds}


def ceilings():
    """Measured ceilings of this device, beside the published peaks (context
    only: the roofline fractions are taken against the published peaks): the
    HBM read rate (moe_probe_read over a 2 GiB buffer, eight times the
    infinity cache), the read rate of scattered expert blocks (moe_probe_gather:
    200 of the 227 bf16 expert blocks of the 256-expert layer, 9.4 MB each,
    that fit in 2 GiB, in a seeded order) and how it grows with the number of
    workgroups reading (one per CU up to 256), the MXFP4 dequantisation stream
    (moe_probe_mxfp4 over 1 GiB of codes and their scales) and the sustained
    bf16 MFMA rate (moe_probe_mfma, 2 waves per SIMD of 8 independent
    16x16x32 chains); best of 5 timed runs each."""
    import torch

    import routed_expert_ffn_moe_amd as moe
    st = torch.cuda.current_stream()

    def best_ms(f):
        f()
        torch.cuda.synchronize()
        b = float("inf")
        for _ in range(5):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(st)
            f()
            e1.record(st)
            e1.synchronize()
            b = min(b, e0.elapsed_time(e1))
        return b

    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    t_read = best_ms(lambda: moe.moe_probe_read(buf))
    # scattered expert blocks: one bf16 expert (gate, up, down) of the
    # 256-expert layer per chunk
    chunk = 3 * 2048 * 768 * 2
    pool_chunks = nbytes // chunk
    import numpy as np
    order = torch.from_numpy(np.random.default_rng(107).permutation(pool_chunks)[:200]
                             .astype(np.int32)).cuda()
    t_gather = best_ms(lambda: moe.moe_probe_gather(buf, chunk, order, 1024))
    per_wg = {}
    few = order[:24].contiguous()
    for wgs in (8, 32, 64, 128, 256, 1024):
        t = best_ms(lambda: moe.moe_probe_gather(buf, chunk, few, wgs))
        per_wg[wgs] = round(few.numel() * chunk / (t * 1e-3) / 1e9, 1)
    del buf
    nblk = (1 << 30) // 16
    codes = torch.full((1 << 30,), 0x3B, dtype=torch.uint8, device="cuda")
    scales = torch.full((nblk,), 120, dtype=torch.uint8, device="cuda")
    sums = torch.empty(1024, dtype=torch.float32, device="cuda")
    t_mx = best_ms(lambda: moe.moe_probe_mxfp4(codes, scales, sums))
    del codes, scales
    waves = 8 * torch.cuda.get_device_properties(0).multi_processor_count
    iters = 20000
    t_mma = best_ms(lambda: moe.moe_probe_mfma(waves, iters))
    return {"hbm_read_GBps": round(nbytes / (t_read * 1e-3) / 1e9, 1),
            "scattered_expert_read_GBps": round(order.numel() * chunk / (t_gather * 1e-3) / 1e9, 1),
            "scattered_read_GBps_by_workgroups": per_wg,
            "mxfp4_dequant_stream_GBps": round((1 << 30) * 17 / 16 / (t_mx * 1e-3) / 1e9, 1),
            "bf16_mfma_TFLOPs": round(waves * iters * 8 * 16384 / (t_mma * 1e-3) / 1e12, 1),
            "probes": "moe_probe_read over 2 GiB; moe_probe_gather, 200 expert blocks of %d B "
                      "(24 for the workgroup counts); moe_probe_mxfp4 over 1 GiB of codes; "
                      "moe_probe_mfma, %d waves x %d rounds" % (chunk, waves, iters)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(wl, seconds):
    """The CPU oracle (as it stands: plain C, fp64, one token at a time, OpenMP
    over tokens) on seeded samples of the workload's tokens, with all host
    threads and with one; each figure the median of three timed samples
    sized to about a third of `seconds`."""
    import numpy as np

    import moe_inputs as mi
    import oracle
    c, lay = wl.c, wl.layers[0]
    h = mi.to_host
    L = oracle.Layer(H=c["H"], E=c["E"], top_k=c["top_k"], I=c["I"], act=c["act"], w=c["w"],
                     router_w=lay.router_w, router_bias=lay.router_bias, w_gate=h(lay.w_gate),
                     w_up=h(lay.w_up), w_down=h(lay.w_down), s_gate=h(lay.s_gate),
                     s_up=h(lay.s_up), s_down=h(lay.s_down), I_shared=c["I_shared"],
                     sh_gate=h(lay.sh_gate), sh_up=h(lay.sh_up), sh_down=h(lay.sh_down))
    x = wl.x_host
    rng = np.random.default_rng(0)
    all_threads = oracle.max_threads()

    def rate(threads, budget):
        oracle.set_threads(threads)
        n = max(1, min(c["T"], threads))
        t0 = time.perf_counter()
        oracle.forward(L, x, np.sort(rng.choice(c["T"], n, replace=False)).astype(np.int32))
        dt = time.perf_counter() - t0
        n = int(min(c["T"], max(n, n * budget / max(dt, 1e-3))))
        runs = []
        for _ in range(3):
            tok = np.sort(rng.choice(c["T"], n, replace=False)).astype(np.int32)
            t0 = time.perf_counter()
            oracle.forward(L, x, tok)
            runs.append(n / (time.perf_counter() - t0))
        return n, sorted(runs)[1], runs

    n_all, v_all, r_all = rate(all_threads, seconds / 6)
    n_one, v_one, r_one = rate(1, seconds / 6)
    oracle.set_threads(all_threads)
    return {"value": round(v_all, 2), "unit": "tokens/s", "cores": all_threads, "kind": "oracle",
            "sample": "median of 3 samples of %d of the %d tokens (seeded), full layer per token, "
                      "%d threads" % (n_all, c["T"], all_threads),
            "one_thread": {"value": round(v_one, 2), "unit": "tokens/s",
                           "sample": "median of 3 samples of %d tokens, 1 thread" % n_one,
                           "runs": [round(v, 2) for v in r_one]},
            "runs": [round(v, 2) for v in r_all],
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}


def describe(wl, wall, stages, steps, graph_wall=None):
    """Throughput, stage times, roofline of the dominant stage and of the
    whole layer for one workload's timing."""
    c = wl.c
    counts = wl.counts()
    fused = stages.get("combine", 0.0) == 0.0
    work = stage_work(c, counts, fused_down_combine=fused)
    dom = max(stages, key=lambda k: stages[k])
    ms_step = wall / steps * 1e3
    gemm = {k: {"us": round(stages[k] * 1e3, 2),
                "frac_hbm": roofline(work, k, stages[k], c["w"])["frac"]
                if work[k][0] else None,
                "frac_mfma_useful": mfma_frac(work, k, stages[k], c["w"])}
            for k in ("gate_up", "down")}
    out = {"tokens_per_s": round(c["T"] / (ms_step / 1e3), 1),
           "us_per_step": round(ms_step * 1e3, 2),
           "weight_sets": len(wl.weights), "experts_touched": work["_Es"],
           "max_rows_per_expert": int(counts.max()),
           "stages_us": {k: round(v * 1e3, 2) for k, v in stages.items()},
           "roofline": dict(roofline(work, dom, stages[dom], c["w"]),
                            traffic=measured_traffic(wl.name, dom)),
           "layer": layer_roofline(work, ms_step, c["w"]),
           "grouped_gemms": gemm,
           "overhead_bytes": work["_overhead"]}
    if graph_wall is not None:
        out["graph_us_per_step"] = round(graph_wall / steps * 1e6, 2)
        out["graph_tokens_per_s"] = round(c["T"] / (graph_wall / steps), 1)
    return out


def decode_stack(name, L, steps, warmup):
    """L MoE layers of the decode workload `name` chained as a model's MoE
    layers run, the output of layer l the input of layer l + 1, each layer
    with its own weights: per-layer time with the L calls launched one after
    the other (eager) and with all of them captured into one HIP graph and
    replayed as one submission."""
    import torch

    import moe_inputs as mi
    import routed_expert_ffn_moe_amd as moe
    wl = Workload(name, wsets=L)
    c = wl.c
    bufs = [wl.x] + [torch.empty_like(wl.x) for _ in range(L)]
    idx = torch.empty((L, c["T"], c["top_k"]), dtype=torch.int32, device="cuda")
    w = torch.empty((L, c["T"], c["top_k"]), dtype=torch.float32, device="cuda")

    def stack():
        for l in range(L):
            moe.moe_forward(wl.shape, wl.weights[l], bufs[l], bufs[l + 1], idx[l], w[l], wl.ws)

    for _ in range(warmup):
        stack()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        stack()
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) / steps
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        stack()
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            stack()
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    graph = (time.perf_counter() - t0) / steps
    del wl, bufs
    torch.cuda.empty_cache()
    return {"workload": mi.cfg(name)["desc"], "layers": L,
            "eager_us_per_layer": round(eager / L * 1e6, 2),
            "graph_us_per_layer": round(graph / L * 1e6, 2),
            "graph_tokens_per_s_per_layer": round(c["T"] / (graph / L), 1)}


SMALL_T = (1, 2, 4, 6, 8, 16, 32, 64)


def small_t_sweep(steps, warmup, Ts=SMALL_T):
    """The MXFP4 decode/verify layer (H=2048, 256 experts top-8, I=768) at
    small T: per-step time, gate+up stage time and its fraction of 8 TB/s,
    weight sets rotated so the weights come from HBM."""
    import moe_inputs as mi
    torch = __import__("torch")
    c0 = mi.cfg("c4_t6")
    wl = Workload("c4_t6", wsets=16, cfg=dict(c0, T=max(Ts)))
    x_all = wl.x
    out = []
    for T in Ts:
        wl.c = dict(c0, T=T)
        wl.x = x_all[:T]
        wl.shape = wl.moe.make_shape(T, c0["H"], c0["E"], c0["top_k"], c0["I"], 0, 0,
                                     c0["act"], c0["w"])
        nb = wl.moe.moe_workspace_bytes(wl.shape)
        if wl.ws.numel() < nb:
            wl.ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        wl.y = torch.empty_like(wl.x)
        wl.idx = torch.empty((T, c0["top_k"]), dtype=torch.int32, device="cuda")
        wl.w = torch.empty((T, c0["top_k"]), dtype=torch.float32, device="cuda")
        n = max(steps, 200)
        wall, stages = wl.time(n, warmup)
        d = describe(wl, wall, stages, n)
        out.append({"T": T, "us_per_step": d["us_per_step"], "tokens_per_s": d["tokens_per_s"],
                    "experts_touched": d["experts_touched"],
                    "gate_up_us": d["stages_us"]["gate_up"],
                    "gate_up_frac_hbm": d["grouped_gemms"]["gate_up"]["frac_hbm"],
                    "layer_frac": d["layer"]["frac"]})
    del wl
    torch.cuda.empty_cache()
    return {"layer": "H=2048 E=256 top-8 I=768, MXFP4 experts, 16 weight sets", "points": out}


SWEEP_T = (128, 256, 512, 1024, 2048, 4096, 8192, 16384, 32768, 65536)


def sweep(steps, warmup, Ts=SWEEP_T):
    """Tokens/s of the T=128 prefill layer (H=2048, 256 experts top-8,
    I=768, bf16, no routing bias) over chunk sizes T, on one weight set and one
    token set (the first T rows of the largest chunk), and the knee of its
    per-token cost: the smallest T whose cost is within 5% of the largest
    chunk's, with the quantum that puts that many tokens on each expert,
    quantum = tokens per expert x E / k."""
    import moe_inputs as mi
    torch = __import__("torch")
    c0 = mi.cfg("c1")
    wl = Workload("c1", wsets=1, cfg=dict(c0, T=max(Ts)))
    x_all = wl.x
    points = []
    for T in Ts:
        wl.c = dict(c0, T=T)
        wl.x = x_all[:T]
        wl.shape = wl.moe.make_shape(T, c0["H"], c0["E"], c0["top_k"], c0["I"], 0, 0,
                                     c0["act"], c0["w"])
        nb = wl.moe.moe_workspace_bytes(wl.shape)
        if wl.ws.numel() < nb:
            wl.ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        wl.y = torch.empty_like(wl.x)
        wl.idx = torch.empty((T, c0["top_k"]), dtype=torch.int32, device="cuda")
        wl.w = torch.empty((T, c0["top_k"]), dtype=torch.float32, device="cuda")
        n = max(5, min(steps, int(4e5 / T)))
        wall, stages = wl.time(n, warmup)
        d = describe(wl, wall, stages, n)
        points.append({"T": T, "tokens_per_s": d["tokens_per_s"], "us_per_step": d["us_per_step"],
                       "us_per_token": round(d["us_per_step"] / T, 4),
                       "tokens_per_expert": T * c0["top_k"] / c0["E"],
                       "experts_touched": d["experts_touched"],
                       "layer_frac": d["layer"]["frac"],
                       "gate_up_frac_hbm": d["grouped_gemms"]["gate_up"]["frac_hbm"],
                       "gate_up_frac_mfma": d["grouped_gemms"]["gate_up"]["frac_mfma_useful"],
                       "bound": d["roofline"]["bound"]})
    del wl
    torch.cuda.empty_cache()
    floor = points[-1]["us_per_token"]
    knee = next(p for p in points if p["us_per_token"] <= 1.05 * floor)
    tpe = knee["tokens_per_expert"]
    return {"layer": "H=2048 E=256 top-8 I=768 bf16, no routing bias", "points": points,
            "knee": {"rule": "smallest T with per-token cost within 5%% of T=%d's" % Ts[-1],
                     "T": knee["T"], "tokens_per_expert": tpe,
                     "quantum_for_layer": int(round(tpe * c0["E"] / c0["top_k"])),
                     "quantum_E256_k6": int(round(tpe * 256 / 6)),
                     "quantum_E128_k8": int(round(tpe * 128 / 8))}}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    # 200 steps: a burst of calls after a synchronisation starts with ~10-20%
    # slower calls for its first few milliseconds (the launch queue has not
    # run ahead yet), which 50 steps of the 0.3 ms layer would still include
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--extra", default="c1,c3,c4_t6,c4_t1,c4_p2048",
                    help="comma-separated secondary workloads ('' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip the chunk-size sweep")
    ap.add_argument("--no-small-sweep", action="store_true",
                    help="skip the small-T sweep of the MXFP4 layer")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the ceiling probes")
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip sampling the clocks with rocm-smi (e.g. under a profiler)")
    ap.add_argument("--stack", type=int, default=16, metavar="L",
                    help="layers of the decode stack timed eager and as one HIP graph (0: skip)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES (calibrates HBM "
                         "byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this layer has no multi-GPU path here "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        src = torch.empty(args.copy_probe, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe, "copies": args.steps}))
        return
    import routed_expert_ffn_moe_amd as moe
    moe.load()
    torch.cuda.set_device(0)
    ceil = None if args.no_ceilings else ceilings()

    wl = Workload(args.workload)
    c = wl.c
    steps = max(args.steps, 200 if c["T"] <= 8 else args.steps)
    wall, stages = wl.time(steps, args.warmup)
    gwall = wl.time_graph(steps, args.warmup) if c["T"] <= 16 else None
    per_call = wl.per_call(steps)

    def busy(done):
        while not done():
            for _ in range(10):
                wl.step()
            torch.cuda.synchronize()
    clocks = None if args.no_clocks else clock_log(busy)
    d = describe(wl, wall, stages, steps, gwall)
    ms_step = wall / steps * 1e3
    out = {
        "metric": METRIC,
        "value": round(c["T"] / (ms_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c["w"],
        "data": "synthetic (seeded inputs, random-init weights)",
        "config": {"workload": c["desc"], "T": c["T"], "H": c["H"], "E": c["E"],
                   "top_k": c["top_k"], "I": c["I"], "I_shared": c["I_shared"],
                   "bias": c["bias"], "experts_touched": d["experts_touched"],
                   "max_rows_per_expert": d["max_rows_per_expert"]},
        "roofline": d["roofline"],
        "layer_roofline": d["layer"],
        "grouped_gemms": d["grouped_gemms"],
        "overhead_bytes": d["overhead_bytes"],
        "stages_us": d["stages_us"],
        "per_call_us": per_call,
        "clocks": clocks,
        "weight_sets": d["weight_sets"],
        "ceilings": ceil,
        "tuning": {k: v for k, v in os.environ.items() if k.startswith("MOE_")},
    }
    if gwall is not None:
        out["graph_us_per_step"] = d["graph_us_per_step"]
    also = {}
    del wl
    torch.cuda.empty_cache()
    import moe_inputs as mi
    for name in [s for s in args.extra.split(",") if s]:
        w2 = Workload(name)
        cc = w2.c
        st = max(args.steps, 200 if cc["T"] <= 8 else args.steps)
        wall2, st2 = w2.time(st, args.warmup)
        g2 = w2.time_graph(st, args.warmup) if cc["T"] <= 16 else None
        also[name] = {"workload": mi.cfg(name)["desc"], **describe(w2, wall2, st2, st, g2),
                      "per_call_us": w2.per_call(st)}
        del w2
        torch.cuda.empty_cache()
    out["also"] = also
    if args.stack:
        out["decode_stack"] = [decode_stack(n, args.stack, 50, 5) for n in ("c4_t1", "c4_t6")]
    if not args.no_small_sweep:
        out["small_T_mxfp4"] = small_t_sweep(args.steps, args.warmup)
    if not args.no_sweep:
        out["sweep"] = sweep(args.steps, args.warmup)
    if not args.no_cpu_baseline:
        wl = Workload(args.workload, keep_rowmajor=True, wsets=1)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
