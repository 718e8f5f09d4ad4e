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


def stage_work(c, counts):
    """Algorithmic bytes and flops of each stage for one call: every operand
    read once, every output written once; expert weights only for the experts
    that received tokens."""
    T, H, E, k, I, Is = c["T"], c["H"], c["E"], c["top_k"], c["I"], c["I_shared"]
    a = 4 if c["act"] == "f32" else 2
    bw = {"f32": 4.0, "bf16": 2.0, "mxfp4": 17.0 / 32.0}[c["w"]]
    Es = int((counts > 0).sum())
    pairs = T * k
    rows = pairs + (T if Is else 0)
    return {
        "router": (T * H * a + E * H * a + (E * 4 if c["bias"] else 0) + pairs * 8,
                   2.0 * T * H * E),
        "permute": (pairs * 4 * 3, 0.0),
        "gate_up": (Es * 2 * I * H * bw + 2 * Is * H * a + T * H * a + pairs * I * a + T * Is * a,
                    4.0 * pairs * H * I + 4.0 * T * H * Is),
        "down": (Es * H * I * bw + H * Is * a + pairs * I * a + T * Is * a + rows * H * a,
                 2.0 * pairs * H * I + 2.0 * T * H * Is),
        "combine": (rows * H * a + T * H * a, float(rows * H)),
        "_Es": Es,
    }


PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")


def kernel_sources_sha1():
    """Digest of the HIP sources: counter readings taken from other sources
    no longer describe the kernels that run."""
    import hashlib
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "routed_expert_ffn_moe_amd", "csrc")
    h = hashlib.sha1()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(f.encode())
            with open(os.path.join(d, f), "rb") as fh:
                h.update(fh.read())
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
    byts, flops = work[stage]
    dur = ms / 1e3
    t_hbm = byts / (PEAK_HBM_GBS * 1e9)
    t_mma = flops / (PEAK_TFLOPS[dtype] * 1e12)
    if t_mma > t_hbm:
        ach = flops / dur / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_TFLOPS[dtype],
                "unit": "TFLOP/s", "frac": round(ach / PEAK_TFLOPS[dtype], 4), "traffic": None,
                "kernel": stage, "avg_us": round(ms * 1e3, 2), "alg_bytes": int(byts),
                "alg_flops": flops}
    ach = byts / dur / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None, "kernel": stage,
            "avg_us": round(ms * 1e3, 2), "alg_bytes": int(byts), "alg_flops": flops}


class Workload:
    def __init__(self, name, wsets=1, dev="cuda", keep_rowmajor=False):
        import torch

        import moe_inputs as mi
        import routed_expert_ffn_moe_amd as moe
        self.torch, self.moe = torch, moe
        self.name = name
        self.keep_rowmajor = keep_rowmajor
        self.c = mi.cfg(name)
        c = self.c
        self.layers = [mi.make_layer(c, dev, s) for s in range(wsets)]
        x = mi.make_x(c)
        self.x_host = x
        t = torch.from_numpy(x)
        self.x = (t.view(torch.int16).view(torch.bfloat16) if c["act"] == "bf16" else t).to(dev)
        self.weights = []
        self._keep = []
        for lay in self.layers:
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
        self.shape = moe.make_shape(c["T"], c["H"], c["E"], c["top_k"], c["I"], c["I_shared"],
                                    0, c["act"], c["w"])
        nb = moe.moe_workspace_bytes(self.shape)
        self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        self.y = torch.empty_like(self.x)
        self.idx = torch.empty((c["T"], c["top_k"]), dtype=torch.int32, device=dev)
        self.w = torch.empty((c["T"], c["top_k"]), dtype=torch.float32, device=dev)
        self.i = 0

    def step(self):
        wt = self.weights[self.i % len(self.weights)]
        self.i += 1
        self.moe.moe_forward(self.shape, wt, self.x, self.y, self.idx, self.w, self.ws)

    def time(self, steps, warmup):
        torch, moe = self.torch, self.moe
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        # per-stage HIP-event times over a second pass of the same steps
        moe.moe_stage_timing_enable(True)
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        ms, n = moe.moe_stage_timing_read()
        moe.moe_stage_timing_enable(False)
        return wall, {k: v / max(n, 1) for k, v in ms.items()}

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


def ceilings():
    """Measured ceilings of this device, beside the published peaks: the HBM
    read rate (moe_probe_read over a 2 GiB buffer, eight times the infinity
    cache) and the sustained bf16 MFMA rate (moe_probe_mfma, 2 waves per SIMD
    of 8 independent 16x16x32 chains); best of 5 timed runs each."""
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
    del buf
    waves = 8 * torch.cuda.get_device_properties(0).multi_processor_count
    iters = 20000
    t_mma = best_ms(lambda: moe.moe_probe_mfma(waves, iters))
    return {"hbm_read_GBps": round(nbytes / (t_read * 1e-3) / 1e9, 1),
            "bf16_mfma_TFLOPs": round(waves * iters * 8 * 16384 / (t_mma * 1e-3) / 1e12, 1),
            "probes": "moe_probe_read over 2 GiB; moe_probe_mfma, %d waves x %d rounds" % (waves, iters)}


def with_ceiling(roof, ceil):
    """The roofline entry plus the fraction of the measured ceiling."""
    m = ceil["hbm_read_GBps"] if roof["bound"] == "hbm" else (
        ceil["bf16_mfma_TFLOPs"] if roof["unit"] == "TFLOP/s" and roof["peak"] == PEAK_TFLOPS["bf16"]
        else None)
    if m:
        roof = dict(roof, measured_ceiling=m, frac_of_measured=round(roof["achieved"] / m, 4))
    return roof


def cpu_baseline(wl, seconds):
    """The CPU oracle (as it stands) on a sample of the workload's tokens."""
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
    n = 16
    t0 = time.perf_counter()
    oracle.forward(L, x, np.sort(rng.choice(c["T"], n, replace=False)).astype(np.int32))
    dt = time.perf_counter() - t0
    n = int(min(c["T"], max(n, n * seconds / max(dt, 1e-3))))
    tok = np.sort(rng.choice(c["T"], n, replace=False)).astype(np.int32)
    t0 = time.perf_counter()
    oracle.forward(L, x, tok)
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(n / dt, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%d of the %d tokens of the workload (seeded), full layer per token, "
                      "%.1f s" % (n, c["T"], dt)}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--extra", default="c1,c3,c4_t6,c4_t1",
                    help="comma-separated secondary workloads ('' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    ceil = ceilings()

    wl = Workload(args.workload)
    wall, stages = wl.time(args.steps, args.warmup)
    c = wl.c
    ms_step = wall / args.steps * 1e3
    counts = wl.counts()
    work = stage_work(c, counts)
    dom = max((k for k in stages), key=lambda k: stages[k])
    out = {
        "metric": METRIC,
        "value": round(c["T"] / (ms_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c["w"] if c["w"] != "bf16" else "bf16",
        "data": "synthetic (seeded inputs, random-init weights)",
        "config": {"workload": c["desc"], "T": c["T"], "H": c["H"], "E": c["E"],
                   "top_k": c["top_k"], "I": c["I"], "I_shared": c["I_shared"],
                   "bias": c["bias"], "experts_touched": work["_Es"],
                   "max_rows_per_expert": int(counts.max())},
        "roofline": with_ceiling(dict(roofline(work, dom, stages[dom], c["w"]),
                                      traffic=measured_traffic(args.workload, dom)), ceil),
        "ceilings": ceil,
        "stages_us": {k: round(v * 1e3, 2) for k, v in stages.items()},
        "tuning": {k: v for k, v in os.environ.items() if k.startswith("MOE_")},
    }
    also = {}
    del wl
    torch.cuda.empty_cache()
    for name in [s for s in args.extra.split(",") if s]:
        import moe_inputs as mi
        cc = mi.cfg(name)
        # weight sets rotated so that the touched weights exceed the MALL
        per_call = cc["top_k"] * cc["T"] * 3 * cc["H"] * cc["I"] * (0.53 if cc["w"] == "mxfp4" else 2)
        wsets = 1 if per_call > 2 * MALL_BYTES else int(min(16, 2 * MALL_BYTES // max(per_call, 1) + 1))
        w2 = Workload(name, wsets=wsets)
        steps = max(args.steps, 200 if cc["T"] <= 8 else args.steps)
        wall2, st2 = w2.time(steps, args.warmup)
        cn = w2.counts()
        wk = stage_work(cc, cn)
        d2 = max(st2, key=lambda k: st2[k])
        entry = {}
        if cc["T"] <= 16:
            gwall = w2.time_graph(steps, args.warmup)
            entry = {"graph_tokens_per_s": round(cc["T"] / (gwall / steps), 1),
                     "graph_us_per_step": round(gwall / steps * 1e6, 2)}
        also[name] = {"workload": cc["desc"], "tokens_per_s": round(cc["T"] / (wall2 / steps), 1),
                      "us_per_step": round(wall2 / steps * 1e6, 2), **entry, "weight_sets": wsets,
                      "experts_touched": wk["_Es"],
                      "stages_us": {k: round(v * 1e3, 2) for k, v in st2.items()},
                      "roofline": with_ceiling(dict(roofline(wk, d2, st2[d2], cc["w"]),
                                                    traffic=measured_traffic(name, d2)), ceil)}
        del w2
        torch.cuda.empty_cache()
    out["also"] = also
    if not args.no_cpu_baseline:
        wl = Workload(args.workload, keep_rowmajor=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
