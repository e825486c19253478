#!/usr/bin/env python3
"""Benchmark of the online INT8 W8A8 hot path on one MI355X.

One step = the decode-shaped dense W8A8 workload: for every M in {1, 2, 4, 8}
the gate_up (K=5120, N=17408) and down (K=8704, N=5120) linears, each as
per-token int8 quant of the bf16 activations followed by the int8 GEMM with
the fp32 epilogue to bf16, through linear_w8a8_packed (weights pre-packed at
load; one or two tokens on the down projection run both in one launch).
`value` is the step's algorithmic bytes over its GPU time (GB/s).

Weights rotate over copies, and the rotation counter belongs to the weight
shape: every launch of a shape takes the next copy, so between two uses of
one copy more than 2 x 256 MB of other weights stream by and every launch
reads its weights from HBM, not from the 256 MB Infinity Cache.

The roofline figure of the dominant kernel (the decode GEMM) comes from a
pass of the same eight GEMMs on prepared codes, bracketed by HIP events on
the launch stream.

Extra cases on the same JSON line (``cases``): every decode shape on its own
(linear and GEMM-only), the small single linear (M=16, K=512, N=256; latency,
no roofline grade), prefill M=4096 TOPS, the routed MoE layer tokens/s at
T in {1, 64, 2048}, and the Hadamard-domain linear at M in {1, 256}, each with
its fraction of the relevant roofline.  The MoE cases rotate over seeded
routing inputs and alternate two copies of the layer's weights.

Timing: the stream is first parked on a short spin kernel while the host
enqueues the timed launches, so HIP events measure GPU time rather than
Python launch overhead.  Times are also reported as median, p10 and p90 over
groups of back-to-back launches (events only between groups).  The shader
clock is sampled (amdsmi) while graph-captured decode steps and prefill
GEMMs replay for about half a second each.  Inputs are hashed (SHA-256 of
the host arrays).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W8A8 GEMM TOPS + HBM GB/s (M=1 & M=4096, % roofline); MoE tokens/s"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
I8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA (5.0 POPS)
MALL_BYTES = 256 << 20     # Infinity Cache
PROBE_ELEMS = 1 << 28      # --probe-copy: 1 GiB of fp32 read and 1 GiB written
DECODE_KERNEL = "k_gemm_skinny"
CASE_GROUPS = ("decode", "small", "prefill", "moe", "rot_moe", "hadamard", "mlp", "kv")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--cases", default="all",
                   help="extra cases on the JSON line: all, none, or a comma list of "
                        + ", ".join(CASE_GROUPS))
    p.add_argument("--no-step", action="store_true",
                   help="skip the decode step and its GEMM pass (value null): for counter "
                        "runs of other cases")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--probe-copy", action="store_true",
                   help="counter runs: time only the decode GEMM pass (no step, value "
                        "null), then a 1 GiB fp32 negation (reads 1 GiB, writes 1 GiB): the "
                        "reference kernel that scales the HBM byte counters")
    p.add_argument("--traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no benchmark: turn two rocprofv3 --pmc runs of this script "
                        "(FETCH_SIZE, then WRITE_SIZE, with --probe-copy) into per-kernel "
                        "HBM bytes; with --traffic-out NAME writes profiles/NAME.json")
    p.add_argument("--traffic-out", default="traffic_decode_gemm")
    return p.parse_args()


def src_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "moe_quant_token_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def src_hash_all() -> str:
    return src_hash(*sorted(n for n in os.listdir(os.path.join(ROOT, "moe_quant_token_amd",
                                                               "csrc"))
                            if n.endswith((".hip", ".h"))))


def sha256_arrays(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(memoryview(a).cast("B"))
    return h.hexdigest()


def pct(vals, q):
    s = sorted(vals)
    if not s:
        return None
    i = min(len(s) - 1, max(0, int(round(q / 100.0 * (len(s) - 1)))))
    return s[i]


class ClockSampler:
    """Shader clock (MHz) sampled through amdsmi in a background thread."""

    def __init__(self):
        self.ok = False
        self.samples = []  # (host time, MHz)
        self._stop = False
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            self._clk = amdsmi.AmdSmiClkType.GFX
            amdsmi.amdsmi_get_clock_info(self._h, self._clk)
            self.ok = True
        except Exception as e:  # noqa: BLE001 - no clock figure rather than no benchmark
            self.err = repr(e)
        if self.ok:
            self._t = threading.Thread(target=self._run, daemon=True)
            self._t.start()

    def _run(self):
        while not self._stop:
            try:
                info = self._smi.amdsmi_get_clock_info(self._h, self._clk)
                self.samples.append((time.perf_counter(), float(info["clk"])))
            except Exception:  # noqa: BLE001
                pass
            time.sleep(0.002)

    def stop(self):
        self._stop = True

    def window(self, t0, t1):
        return [v for t, v in self.samples if t0 <= t <= t1]


class GpuTimer:
    """Event timing with the stream parked behind a spin kernel while the host enqueues."""

    def __init__(self, torch, clock: ClockSampler):
        self.torch = torch
        self.clock = clock
        self.busy = []  # host-time windows of the timed regions
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        torch.cuda.synchronize()
        s.record()
        torch.cuda._sleep(2_000_000)
        e.record()
        torch.cuda.synchronize()
        self.ms_per_cycle = max(s.elapsed_time(e) / 2_000_000, 1e-9)
        self.enqueue_bound = False

    def park(self, ms: float):
        self.torch.cuda._sleep(int(ms / self.ms_per_cycle))

    def run(self, fn, iters: int, park_ms: float = 100.0, groups: int = 1):
        """Run fn(i) for i < iters, with HIP events only at the boundaries of
        `groups` equal runs of launches (an event between every two launches
        would add its own gap to short kernels).  Returns (total GPU ms from
        the first launch to the last, per-launch GPU ms of each group)."""
        torch = self.torch
        groups = max(1, min(groups, iters))
        bounds = [round(g * iters / groups) for g in range(groups + 1)]
        torch.cuda.synchronize()
        self.park(park_ms)
        t0 = time.perf_counter()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(groups + 1)]
        evs[0].record()
        g = 1
        for i in range(iters):
            fn(i)
            if i + 1 == bounds[g]:
                evs[g].record()
                g += 1
        if (time.perf_counter() - t0) * 1e3 > park_ms:
            self.enqueue_bound = True
        torch.cuda.synchronize()
        # the timed launches start once the spin kernel ends
        self.busy.append((t0 + park_ms * 1e-3, time.perf_counter()))
        total = evs[0].elapsed_time(evs[groups])
        per = [evs[k].elapsed_time(evs[k + 1]) / (bounds[k + 1] - bounds[k])
               for k in range(groups)]
        return total, per

    def stats_us(self, per_ms):
        return {"median_us": round(pct(per_ms, 50) * 1e3, 2),
                "p10_us": round(pct(per_ms, 10) * 1e3, 2),
                "p90_us": round(pct(per_ms, 90) * 1e3, 2)}


def linear_bytes(M, N, K, bf16_in: bool) -> int:
    a = M * K * 2 if bf16_in else M * K + 4 * M
    return N * K + 4 * N + a + 2 * M * N


def _counter_rows(d: str, counter: str):
    """(kernel name, value) per dispatch from a rocprofv3 --pmc csv directory."""
    import csv
    import glob

    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def traffic_from_counters(fetch_dir: str, write_dir: str, out_name: str) -> None:
    """HBM bytes per launch of every kernel from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch).  Each counter is scaled by what it reads for the probe kernel, a
    plain fp32 negation over 1 GiB (1 GiB fetched, 1 GiB written), so the
    figures are bytes of the same kind as the algorithmic ones."""
    # src_hash: the decode GEMM's source (its figure is void once that changes);
    # src_hash_all: every kernel source, for the other kernels' figures
    out = {"src_hash": src_hash("gemm_skinny.hip"), "src_hash_all": src_hash_all(),
           "kernels": {}}
    for key, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _counter_rows(d, counter)
        probe = [v for n, v in rows if "neg" in n]
        if not probe:
            raise SystemExit(f"{counter}: no probe dispatch")
        scale = float(PROBE_ELEMS * 4) / (max(probe) * 1024.0)
        out[key + "_scale"] = scale
        per = {}
        for n, v in rows:
            n = n[5:] if n.startswith("void ") else n
            if "neg" in n or not n.startswith("w8a8::"):
                continue
            name = n.split("(")[0]
            per.setdefault(name, []).append(v)
        for name, vals in per.items():
            k = out["kernels"].setdefault(name, {})
            k[key + "_dispatches"] = len(vals)
            k[key + "_kib_avg_raw"] = sum(vals) / len(vals)
            k[key + "_bytes"] = sum(vals) / len(vals) * 1024.0 * scale
    for k in out["kernels"].values():
        k["bytes_per_launch"] = k.get("fetch_bytes", 0.0) + k.get("write_bytes", 0.0)
    dec = [v for n, v in out["kernels"].items() if DECODE_KERNEL in n]
    if dec:
        out["kernel"] = DECODE_KERNEL
        out["bytes_per_launch"] = sum(v["bytes_per_launch"] for v in dec) / len(dec)
    path = os.path.join(ROOT, "profiles", out_name + ".json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def main():
    args = parse()
    if args.traffic:
        traffic_from_counters(*args.traffic, args.traffic_out)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the "
              "kernels run on one GPU's share of a layer; nothing here spans GPUs)",
              file=sys.stderr)
        sys.exit(2)
    groups = set(CASE_GROUPS) if args.cases == "all" else \
        set() if args.cases == "none" else set(args.cases.split(","))
    unknown = groups - set(CASE_GROUPS)
    if unknown:
        raise SystemExit(f"unknown case groups: {sorted(unknown)}")

    import numpy as np
    import torch

    import moe_quant_token_amd as mq
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    clock = ClockSampler()
    timer = GpuTimer(torch, clock)

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).to(dev)

    # ------------------------------------------------------------ decode step
    shapes = []
    hashes = {}
    for si, (K, N, name) in enumerate(synth.DECODE_SHAPES):
        Wh = synth.weights(synth.decode_linear(1, si)["wkey"], N, K)
        hashes[f"decode_{name}_weights_fp32"] = sha256_arrays(Wh)
        W = torch.from_numpy(Wh).to(dev)
        qw, sw = mq.quant_per_token_i8(W)          # weight preparation, untimed
        del W, Wh
        qw = mq.pack_weights(qw)                   # MFMA tile layout, untimed
        wbytes = N * K + 4 * N
        ncopy = max(2, math.ceil(2 * MALL_BYTES / wbytes) + 1)
        copies = [(qw, sw)] + [(qw.clone(), sw.clone()) for _ in range(ncopy - 1)]
        shapes.append(dict(K=K, N=N, name=name, copies=copies, use=0))
    calls = []
    xs_h = []
    for M in synth.DECODE_M:
        for si, sh in enumerate(shapes):
            cfg = synth.decode_linear(M, si)
            xh = synth.activations(cfg["xkey"], M, sh["K"], cfg["n_outliers"],
                                   cfg["outlier_scale"])
            xs_h.append(xh)
            x = bf16_dev(xh)
            q, s = mq.quant_per_token_i8(x)  # codes for the GEMM-only pass, untimed
            y = torch.empty((M, sh["N"]), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(mq.linear_w8a8_workspace_bytes(M, sh["N"], sh["K"]),
                             dtype=torch.uint8, device=dev)
            calls.append(dict(M=M, sh=sh, x=x, q=q, s=s, y=y, ws=ws))
    hashes["decode_activations_bf16"] = sha256_arrays(*xs_h)
    step_bytes = sum(linear_bytes(c["M"], c["sh"]["N"], c["sh"]["K"], True) for c in calls)
    gemm_bytes = sum(linear_bytes(c["M"], c["sh"]["N"], c["sh"]["K"], False) for c in calls)

    L = mq.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream

    def weights(sh):
        # the next copy of this weight shape, whatever M the launch has
        qw, sw = sh["copies"][sh["use"] % len(sh["copies"])]
        sh["use"] += 1
        return qw, sw

    def linear_call(c):
        sh = c["sh"]
        qw, sw = weights(sh)
        st = L.linear_w8a8_packed(c["x"].data_ptr(), c["M"], sh["K"], sh["K"], qw.data_ptr(),
                                  sw.data_ptr(), sh["N"], c["y"].data_ptr(), sh["N"],
                                  c["ws"].data_ptr(), c["ws"].numel(), stream)
        if st != 0:
            raise RuntimeError(f"linear_w8a8_packed failed: {st}")

    def gemm_call(c, warm=False):
        sh = c["sh"]
        qw, sw = sh["copies"][0] if warm else weights(sh)
        st = L.gemm_w8a8_packed(c["q"].data_ptr(), c["s"].data_ptr(), c["M"], sh["K"], sh["K"],
                                qw.data_ptr(), sw.data_ptr(), sh["N"], c["y"].data_ptr(),
                                sh["N"], None, 0, stream)
        if st != 0:
            raise RuntimeError(f"gemm_w8a8_packed failed: {st}")

    def step(i):
        # one decode step: the linear entry point on each of the eight linears
        # (quant + GEMM, or both in one launch where the library does that)
        for c in calls:
            linear_call(c)

    def gemm_pass(i):
        # the dominant kernel alone: the eight decode GEMMs on prepared codes
        for c in calls:
            gemm_call(c)

    out = {
        "metric": METRIC,
        "value": None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {
            "workload": "decode dense W8A8 linear: M in {1,2,4,8} x (gate_up K=5120 N=17408, "
                        "down K=8704 N=5120), bf16 in -> per-token int8 quant -> int8 GEMM -> "
                        "bf16 out",
            "weight_copies": {sh["name"]: len(sh["copies"]) for sh in shapes},
            "step_bytes": step_bytes,
        },
    }

    if not args.no_step:
        counters_only = args.probe_copy
        for i in range(args.warmup):
            if not counters_only:
                step(i)
            gemm_pass(i)
        torch.cuda.synchronize()
        if not counters_only:
            total_ms, step_ms = timer.run(step, args.steps, groups=max(1, args.steps // 4))
            ms_per_step = total_ms / args.steps
            out["ms_per_step"] = round(ms_per_step, 5)
            out["value"] = round(step_bytes / (ms_per_step * 1e-3) / 1e9, 2)
            out["step_time"] = timer.stats_us(step_ms)
        # the dominant kernel: HIP events around every GEMM launch of the pass,
        # on the stream the kernels run on
        n_gemm = len(calls) * args.steps
        gemm_total, gemm_each = timer.run(lambda i: gemm_call(calls[i % len(calls)]), n_gemm,
                                          groups=args.steps)
        gemm_avg_us = gemm_total * 1e3 / n_gemm
        achieved = (gemm_bytes / len(calls)) / (gemm_avg_us * 1e-6) / 1e9
        traffic = None
        tpath = os.path.join(ROOT, "profiles", "traffic_decode_gemm.json")
        if os.path.exists(tpath):
            with open(tpath) as f:
                tj = json.load(f)
            if tj.get("src_hash") == src_hash("gemm_skinny.hip"):
                traffic = tj.get("bytes_per_launch")
        out["roofline"] = {
            "kernel": "k_gemm_skinny (decode weight-streaming int8 GEMM)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(gemm_avg_us, 3),
            "launch_us": timer.stats_us(gemm_each),
            "bytes_per_launch": gemm_bytes / len(calls),
        }

    # shader clock while graph-captured decode steps replay
    clocks = {}
    if not args.no_step and not args.probe_copy and clock.ok:
        def capture_steps():
            for c in calls:
                qw, sw = weights(c["sh"])
                mq.linear_w8a8_packed(c["x"], qw, sw, c["sh"]["N"], y=c["y"], ws=c["ws"])
        probe = clock_probe(torch, clock, lambda: [capture_steps() for _ in range(8)], 0.5)
        probe["step_us"] = round(probe.pop("replay_us") / 8, 2)
        clocks["decode_step_graph"] = probe

    # ------------------------------------------------------------ what HBM delivers
    # torch's own copy and sum kernels over 1 GiB buffers, and the library's
    # streaming-read kernel over each decode shape's weight bytes: the rates
    # this GPU delivers at this moment, beside which the roofline fractions
    # (against the published 8 TB/s) can be read
    if not args.probe_copy:
        out["hbm_stream"] = stream_ceiling(torch, timer, mq, shapes)

    # ------------------------------------------------------------ extra cases
    cases = {}
    if "decode" in groups:
        cases.update(decode_cases(calls, linear_call, gemm_call, timer))
    if "small" in groups:
        cases.update(small_case(torch, np, mq, synth, dev, timer, bf16_dev, hashes))
    if "prefill" in groups:
        cases.update(prefill_cases(torch, np, mq, synth, dev, timer, bf16_dev, hashes))
    if "moe" in groups:
        cases.update(moe_cases(torch, np, mq, synth, dev, timer, bf16_dev, hashes))
    if "rot_moe" in groups:
        cases.update(rot_moe_cases(torch, np, mq, synth, dev, timer, bf16_dev, hashes))
    if "hadamard" in groups:
        cases.update(hadamard_cases(torch, np, mq, synth, dev, timer, bf16_dev, hashes))
    if "mlp" in groups:
        cases.update(mlp_cases(torch, np, mq, synth, dev, timer, bf16_dev, hashes))
    if "kv" in groups:
        cases.update(kv_cases(torch, np, mq, synth, dev, timer, bf16_dev, hashes))
    if cases and "hbm_stream" in out:
        annotate_stream(cases, out["hbm_stream"]["stream_read"])
    if cases:
        out["cases"] = cases
    if timer.enqueue_bound:
        out["enqueue_bound_warning"] = True
    if "prefill" in groups and clock.ok:
        clocks["prefill_gemm_graph"] = prefill_clock_probe(torch, mq, synth, dev, clock)
    clock.stop()
    if clock.ok:
        busy = [v for t0, t1 in timer.busy for v in clock.window(t0, t1)]
        out["sclk_mhz"] = {"timed_regions": {"median": pct(busy, 50), "samples": len(busy)},
                           **clocks,
                           "source": "amdsmi GFX clock, sampled every ~2 ms"}
    else:
        out["sclk_mhz"] = None
    out["inputs_sha256"] = hashes

    if args.probe_copy:
        a = torch.zeros(PROBE_ELEMS, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b

    # ------------------------------------------------------------ CPU baseline
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(np, synth, args.cpu_seconds, step_bytes)

    print(json.dumps(out), flush=True)


def stream_ceiling(torch, timer, mq, shapes):
    """Streaming rates: torch's copy (1 GiB read + 1 GiB written) and sum (1 GiB
    read) kernels, median of 10 launches each, in GB/s of bytes moved; and the
    library's streaming-read kernel (w8a8_stream_read) reading exactly the
    weight bytes of each decode shape with the decode GEMM's access pattern
    (one workgroup per 16 weight rows, chunk = 16 K bytes), rotating over
    copies as the step does, median of 48 launches, plus one 713 MB read."""
    n = 1 << 28  # fp32 elements: 1 GiB
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    r = torch.empty((), dtype=torch.float32, device="cuda")
    b.copy_(a)
    torch.sum(a, dim=(0,), out=r)
    _, cp = timer.run(lambda i: b.copy_(a), 10, groups=10)
    _, sm = timer.run(lambda i: torch.sum(a, dim=(0,), out=r), 10, groups=10)
    res = {"copy_gbs": round(2 * 4 * n / (pct(cp, 50) * 1e-3) / 1e9, 1),
           "read_gbs": round(4 * n / (pct(sm, 50) * 1e-3) / 1e9, 1),
           "source": "torch copy_ and sum over 1 GiB fp32, median of 10"}
    del a, b, r
    # the streaming-read kernel over one buffer sliced like the weight copies
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    big = max(sh["N"] * sh["K"] for sh in shapes) * 8
    buf = torch.zeros(big, dtype=torch.int8, device="cuda")
    probe = {}
    for sh in shapes:
        nbytes, chunk = sh["N"] * sh["K"], 16 * sh["K"]
        nslice = big // nbytes
        views = [buf[i * nbytes:(i + 1) * nbytes] for i in range(nslice)]
        for i in range(nslice):
            mq.stream_read(views[i], chunk, sink)
        _, each = timer.run(lambda i: mq.stream_read(views[i % nslice], chunk, sink), 48,
                            groups=8)
        med = pct(each, 50)
        probe[sh["name"]] = {"bytes": nbytes, "chunk": chunk, "median_us": round(med * 1e3, 2),
                             "gbs": round(nbytes / (med * 1e-3) / 1e9, 1)}
    # reads the size of one-token launches: a single-token MoE gemm1 (8 experts'
    # 1024 x 2048 codes, 32 KiB a workgroup) and gemm2 (8 x 2048 x 512, 8 KiB a
    # workgroup), alone and as two launches back to back, the ceiling of a
    # two-launch single-token layer; the first alone is also the size of the
    # one-token Hadamard linear's weights (8192 x 2048)
    small = {"t1_gemm1": (8 * 1024 * 2048, 16 * 2048), "t1_gemm2": (8 * 2048 * 512, 16 * 512)}
    sviews = {}
    for name, (nbytes, chk) in small.items():
        nslice = big // nbytes
        sviews[name] = ([buf[i * nbytes:(i + 1) * nbytes] for i in range(nslice)], chk)
        vs = sviews[name][0]
        _, each = timer.run(lambda i: mq.stream_read(vs[i % len(vs)], chk, sink), 48, groups=8)
        med = pct(each, 50)
        probe[name] = {"bytes": nbytes, "chunk": chk, "median_us": round(med * 1e3, 2),
                       "gbs": round(nbytes / (med * 1e-3) / 1e9, 1)}
    v1, c1 = sviews["t1_gemm1"]
    v2, c2 = sviews["t1_gemm2"]

    def pair(i):
        mq.stream_read(v1[i % len(v1)], c1, sink)
        mq.stream_read(v2[i % len(v2)], c2, sink)

    _, each = timer.run(pair, 48, groups=8)
    probe["t1_two_launches"] = {"bytes": small["t1_gemm1"][0] + small["t1_gemm2"][0],
                                "median_us": round(pct(each, 50) * 1e3, 2)}
    chunk = 80 * 1024
    whole = big // chunk * chunk
    _, each = timer.run(lambda i: mq.stream_read(buf[:whole], chunk, sink), 10, groups=10)
    probe["whole_buffer"] = {"bytes": whole, "chunk": chunk,
                             "median_us": round(pct(each, 50) * 1e3, 2),
                             "gbs": round(whole / (pct(each, 50) * 1e-3) / 1e9, 1)}
    res["stream_read"] = probe
    del buf, sink
    torch.cuda.empty_cache()
    return res


def annotate_stream(cases, probe):
    """Beside each weight-streaming case, the time the streaming-read kernel
    takes for the same weight bytes in the same number of launches (measured
    in this run), and the case's time as a fraction of it: how close the
    kernel comes to what a launch of that size can stream on this GPU."""
    def put(name, ref):
        c = cases.get(name)
        if c is None or ref not in probe:
            return
        t = c["median_us"] if "median_us" in c else None
        if t:
            c["stream_ceiling_us"] = probe[ref]["median_us"]
            c["frac_stream"] = round(probe[ref]["median_us"] / t, 4)
    for name in list(cases):
        if name.startswith("decode_gate_up_") and not name.endswith("_warm"):
            put(name, "gate_up")
        elif name.startswith("decode_down_") and not name.endswith("_warm"):
            put(name, "down")
    put("moe_T1", "t1_two_launches")
    put("rot_moe_T1_routed", "t1_two_launches")
    put("fwht128_g256_M1_K2048_N8192", "t1_gemm1")


def clock_probe(torch, clock, capture, seconds):
    """Capture `capture()` into a graph, replay it for about `seconds` of GPU
    time while the sampler records the shader clock; returns the clock's
    median / p10 / p90 over that window and the GPU time of one replay."""
    g = torch.cuda.CUDAGraph()
    capture()  # eager warm-up
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        capture()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    one_ms = max(a.elapsed_time(b), 1e-3)
    n = max(1, int(seconds * 1e3 / one_ms))
    t0 = time.perf_counter()
    a.record()
    for _ in range(n):
        g.replay()
    b.record()
    while not b.query():
        time.sleep(0.005)
    t1 = time.perf_counter()
    vals = clock.window(t0, t1)
    del g
    return {"median": pct(vals, 50), "p10": pct(vals, 10), "p90": pct(vals, 90),
            "samples": len(vals), "replay_us": round(a.elapsed_time(b) * 1e3 / n, 2),
            "replays": n}


def prefill_clock_probe(torch, mq, synth, dev, clock):
    """Shader clock under the prefill GEMM (4096 x 5120 x 17408, random int8
    codes from the benchmark's inputs), replayed from a graph."""
    cfg = synth.prefill_linear(17408)
    M, K, N = cfg["M"], cfg["K"], cfg["N"]
    qw, sw = mq.quant_per_token_i8(torch.from_numpy(synth.weights(cfg["wkey"], N, K)).to(dev))
    qw = mq.pack_weights(qw)
    xb = synth.activations(cfg["xkey"], M, K, cfg["n_outliers"], cfg["outlier_scale"])
    import numpy as np
    x = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).to(dev)
    q, s = mq.quant_per_token_i8(x)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, mq.gemm_w8a8_workspace_bytes(M, N, K)), dtype=torch.uint8, device=dev)
    r = clock_probe(torch, clock, lambda: mq.gemm_w8a8_packed(q, s, qw, sw, N, y=y, ws=ws), 0.5)
    r["gemm_us"] = r.pop("replay_us")
    del qw, sw, x, q, s, y, ws
    torch.cuda.empty_cache()
    return r


def decode_cases(calls, linear_call, gemm_call, timer):
    """Every decode linear on its own: the linear entry point and the GEMM on
    prepared codes, 48 launches each (weights rotating as in the step)."""
    res = {}
    it = 48
    for c in calls:
        sh = c["sh"]
        M, K, N = c["M"], sh["K"], sh["N"]
        for kind, fn, bf16_in in (("linear", linear_call, True), ("gemm", gemm_call, False)):
            for i in range(4):
                fn(c)
            _, each = timer.run(lambda i: fn(c), it, groups=8)
            med = pct(each, 50)
            nbytes = linear_bytes(M, N, K, bf16_in)
            res[f"decode_{sh['name']}_M{M}_{kind}"] = {
                **timer.stats_us(each),
                "gbs": round(nbytes / (med * 1e-3) / 1e9, 1),
                "frac_hbm": round(nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "alg_bytes": nbytes,
            }
        if M == 1:
            # warm: one weight copy over and over, so the weights sit in the
            # 256 MB Infinity Cache (labelled; not an HBM figure)
            fn = lambda i: gemm_call(c, warm=True)
            for i in range(4):
                fn(i)
            _, each = timer.run(fn, it, groups=8)
            med = pct(each, 50)
            nbytes = linear_bytes(M, N, K, False)
            res[f"decode_{sh['name']}_M{M}_gemm_warm"] = {
                **timer.stats_us(each),
                "gbs": round(nbytes / (med * 1e-3) / 1e9, 1),
                "note": "one weight copy (Infinity Cache resident); not an HBM rate",
            }
    return res


def small_case(torch, np, mq, synth, dev, timer, bf16_dev, hashes):
    """The small single linear (M=16, K=512, N=256): 0.15 MB of traffic, so its
    time is launch latency; reported as time only."""
    cfg = synth.small_linear()
    M, K, N = cfg["M"], cfg["K"], cfg["N"]
    xh = synth.activations(cfg["xkey"], M, K, cfg["n_outliers"], cfg["outlier_scale"])
    Wh = synth.weights(cfg["wkey"], N, K)
    hashes["small_linear"] = sha256_arrays(xh, Wh)
    qw, sw = mq.quant_per_token_i8(torch.from_numpy(Wh).to(dev))
    qp = mq.pack_weights(qw)
    x = bf16_dev(xh)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(mq.linear_w8a8_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev)
    for i in range(4):
        mq.linear_w8a8_packed(x, qp, sw, N, y=y, ws=ws)
    _, each = timer.run(lambda i: mq.linear_w8a8_packed(x, qp, sw, N, y=y, ws=ws), 64,
                        groups=8)
    return {f"small_linear_M{M}_K{K}_N{N}": {**timer.stats_us(each),
                                             "note": "latency-bound (0.15 MB); time only"}}


def prefill_cases(torch, np, mq, synth, dev, timer, bf16_dev, hashes):
    res = {}
    for N in (5120, 17408):
        cfg = synth.prefill_linear(N)
        M, K = cfg["M"], cfg["K"]
        Wh = synth.weights(cfg["wkey"], N, K)
        xh = synth.activations(cfg["xkey"], M, K, cfg["n_outliers"], cfg["outlier_scale"])
        hashes[f"prefill_N{N}"] = sha256_arrays(xh, Wh)
        W = torch.from_numpy(Wh).to(dev)
        qw, sw = mq.quant_per_token_i8(W)
        del W, Wh
        qw = mq.pack_weights(qw)
        # weight copies rotate so each launch reads its weights from HBM, not
        # from the Infinity Cache
        ncopy = max(2, math.ceil(2 * MALL_BYTES / (N * K)) + 1)
        copies = [(qw, sw)] + [(qw.clone(), sw.clone()) for _ in range(ncopy - 1)]
        x = bf16_dev(xh)
        q, s = mq.quant_per_token_i8(x)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(mq.linear_w8a8_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev)
        ws_g = torch.empty(max(1, mq.gemm_w8a8_workspace_bytes(M, N, K)), dtype=torch.uint8,
                           device=dev)
        for i in range(2):
            mq.gemm_w8a8_packed(q, s, *copies[-1 - i], N, y=y, ws=ws_g)
        it = 10

        def gemm(i):
            w, sc = copies[i % ncopy]
            mq.gemm_w8a8_packed(q, s, w, sc, N, y=y, ws=ws_g)

        def linear(i):
            w, sc = copies[i % ncopy]
            mq.linear_w8a8_packed(x, w, sc, N, y=y, ws=ws)

        _, eg = timer.run(gemm, it, groups=it)
        _, el = timer.run(linear, it, groups=it)
        t_g, t_l = pct(eg, 50), pct(el, 50)
        ops = 2.0 * M * N * K
        res[f"prefill_M{M}_K{K}_N{N}"] = {
            "gemm": timer.stats_us(eg),
            "gemm_tops": round(ops / (t_g * 1e-3) / 1e12, 1),
            "gemm_frac_mfma": round(ops / (t_g * 1e-3) / 1e12 / I8_PEAK_TOPS, 4),
            "linear_bf16": timer.stats_us(el),
            "linear_bf16_tops": round(ops / (t_l * 1e-3) / 1e12, 1),
            "linear_frac_mfma": round(ops / (t_l * 1e-3) / 1e12 / I8_PEAK_TOPS, 4),
            "weight_copies": ncopy,
        }
        if N == 5120:
            # the per-token quantiser alone on the 4096 x 5120 activations:
            # cold (the rows rotate over copies beyond the Infinity Cache) and
            # warm (one copy, as when the producing op just wrote them)
            xcopies = [x] + [x.clone() for _ in range(math.ceil(2 * MALL_BYTES / (M * K * 2)))]
            qq = torch.empty((M, K), dtype=torch.int8, device=dev)
            ss = torch.empty((M,), dtype=torch.float32, device=dev)
            for xc in xcopies:
                mq.quant_per_token_i8(xc, qq, ss)
            qbytes = M * K * 2 + M * K + 4 * M
            for tag, fn in (("", lambda i: mq.quant_per_token_i8(xcopies[i % len(xcopies)], qq,
                                                                  ss)),
                            ("_warm", lambda i: mq.quant_per_token_i8(x, qq, ss))):
                _, eq = timer.run(fn, 40, groups=8)
                tq = pct(eq, 50)
                res[f"quant_M{M}_K{K}{tag}"] = {
                    **timer.stats_us(eq), "alg_bytes": qbytes,
                    "gbs": round(qbytes / (tq * 1e-3) / 1e9, 1),
                    "frac_hbm": round(qbytes / (tq * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "input_copies": len(xcopies) if not tag else 1}
            del xcopies, qq, ss
        del qw, sw, x, q, s, y, ws, ws_g, copies
        torch.cuda.empty_cache()
    return res


def moe_cases(torch, np, mq, synth, dev, timer, bf16_dev, hashes):
    cfg = synth.moe(1)
    E, H, I, k = cfg["E"], cfg["H"], cfg["I"], cfg["k"]
    w13 = torch.empty((E, 2 * I, H), dtype=torch.int8, device=dev)
    s13 = torch.empty((E, 2 * I), dtype=torch.float32, device=dev)
    w2 = torch.empty((E, H, I), dtype=torch.int8, device=dev)
    s2 = torch.empty((E, H), dtype=torch.float32, device=dev)
    wh = hashlib.sha256()
    for e in range(E):  # weight preparation on the GPU (untimed)
        ah = synth.expert_weights(cfg["wkey"], e, 2 * I, H, synth.T_W)
        bh = synth.expert_weights(cfg["wkey"], e, H, I, synth.T_W2)
        wh.update(memoryview(ah).cast("B"))
        wh.update(memoryview(bh).cast("B"))
        mq.quant_per_token_i8(torch.from_numpy(ah).to(dev), q=w13[e], s=s13[e])
        mq.quant_per_token_i8(torch.from_numpy(bh).to(dev), q=w2[e], s=s2[e])
    hashes["moe_weights_fp32"] = wh.hexdigest()
    w13, w2 = mq.pack_moe_weights(w13, w2)  # MFMA tile layout, untimed
    # two copies of the layer's weights, used alternately, and routing inputs
    # rotating over seeded sets: a call reuses an expert's weights only after
    # far more than the 256 MB Infinity Cache has streamed by
    copies = [(w13, s13, w2, s2), (w13.clone(), s13.clone(), w2.clone(), s2.clone())]
    res = {}
    for T, nsets, it in ((1, 64, 64), (64, 4, 20), (2048, 2, 10)):
        c = synth.moe(T)
        ws = torch.empty(mq.moe_w8a8_workspace_bytes(T, H, E, I, k), dtype=torch.uint8,
                         device=dev)
        sets = []
        ih = hashlib.sha256()
        for r in range(nsets):
            key = c["xkey"] if r == 0 else (*c["xkey"], r)
            xh = synth.activations(key, T, H, 0, 1.0)
            lh = synth.router_logits(key, T, E)
            ih.update(memoryview(xh).cast("B"))
            ih.update(memoryview(lh).cast("B"))
            x = bf16_dev(xh)
            logits = torch.from_numpy(lh).to(dev)
            ids = torch.empty((T, k), dtype=torch.int32, device=dev)
            wt = torch.empty((T, k), dtype=torch.float32, device=dev)
            out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            sets.append((x, logits, ids, wt, out))
        hashes[f"moe_T{T}_inputs"] = ih.hexdigest()

        def fn(i):
            x, logits, ids, wt, out = sets[i % nsets]
            a13, b13, a2, b2 = copies[i % len(copies)]
            mq.moe_w8a8_forward(x, logits, a13, b13, a2, b2, k, topk_ids=ids, topk_w=wt,
                                out=out, ws=ws, packed=True)

        for r in range(nsets):  # every set routed once (ids filled), untimed
            fn(r)
        _, each = timer.run(fn, it, groups=min(it, 8))
        t = pct(each, 50)
        touched = sum(int(torch.unique(st[2]).numel()) for st in sets) / nsets
        nbytes = touched * (2 * I * H + H * I + 4 * (2 * I + H)) + T * H * 2 + T * E * 4 + \
            T * H * 2
        ops = 2.0 * T * k * (2 * I * H + H * I)
        res[f"moe_T{T}"] = {
            **timer.stats_us(each),
            "tokens_per_s": round(T / (t * 1e-3), 1),
            "experts_touched": round(touched, 1),
            "alg_bytes": int(nbytes),
            "gbs": round(nbytes / (t * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "tops": round(ops / (t * 1e-3) / 1e12, 2),
            "routing_sets": nsets,
            "weight_copies": len(copies),
        }
    del copies
    return res


def rot_moe_cases(torch, np, mq, synth, dev, timer, bf16_dev, hashes):
    """The MoE layer in the Hadamard domain at the routed-MoE shapes (256
    experts, top-8, hidden 2048, expert and shared intermediate 512): the bf16
    router gate, the shared expert (g256 gate/up, g128 down) and the routed
    experts on the rotated grid (g128 bf16 scales) with the shared term in the
    combine.  Each piece is timed alone, the three in sequence ("layer"), and the
    router followed by the one-call routed layer with its shared expert
    ("layer_one_call": one token runs it in two launches).
    HBM-graded on the weights the call touches plus activations in and out."""
    cfg = synth.moe(1)
    E, H, I, k = cfg["E"], cfg["H"], cfg["I"], cfg["k"]
    Is = I
    w13 = torch.empty((E, 2 * I, H), dtype=torch.int8, device=dev)
    s13 = torch.empty((E, 2 * I, H // 128), dtype=torch.bfloat16, device=dev)
    w2 = torch.empty((E, H, I), dtype=torch.int8, device=dev)
    s2 = torch.empty((E, H, I // 128), dtype=torch.bfloat16, device=dev)
    wh = hashlib.sha256()
    for e in range(E):  # rotated weight preparation on the GPU (untimed)
        ah = synth.expert_weights(cfg["wkey"], e, 2 * I, H, synth.T_W)
        bh = synth.expert_weights(cfg["wkey"], e, H, I, synth.T_W2)
        wh.update(memoryview(ah).cast("B"))
        wh.update(memoryview(bh).cast("B"))
        w13[e], s13[e] = mq.fwht128_weight_prep_g128(torch.from_numpy(ah).to(dev))
        w2[e], s2[e] = mq.fwht128_weight_prep_g128(torch.from_numpy(bh).to(dev))
    w13, w2 = mq.pack_moe_weights(w13, w2)
    gh = synth.weights((101, 0), 2 * Is, H)
    dh = synth.weights((101, 0), H, Is, tensor_id=synth.T_W2)
    rh = synth.to_bf16_bits(synth.weights((101, 1), E, H))
    wh.update(memoryview(gh).cast("B"))
    wh.update(memoryview(dh).cast("B"))
    wh.update(memoryview(rh).cast("B"))
    hashes["rot_moe_weights_fp32"] = wh.hexdigest()
    qgu, su8, sgu = mq.fwht128_weight_prep_g256(torch.from_numpy(gh).to(dev))
    qd, sd = mq.fwht128_weight_prep_g128(torch.from_numpy(dh).to(dev))
    shared_w = (mq.pack_weights(qgu), su8, sgu, mq.pack_weights(qd), sd)
    wg = bf16_dev(rh)
    copies = [(w13, s13, w2, s2), (w13.clone(), s13.clone(), w2.clone(), s2.clone())]
    expert_bytes = 2 * I * H + H * I + 2 * (2 * I * H // 128 + H * I // 128)
    shared_bytes = 2 * Is * H + 2 * Is * H // 256 + 4 * Is + H * Is + 2 * H * Is // 128
    router_bytes = E * H * 2
    res = {}
    for T, nsets, it in ((1, 64, 64), (64, 4, 20), (2048, 2, 10)):
        c = synth.moe(T)
        ws = torch.empty(mq.moe_w8a8_workspace_bytes(T, H, E, I, k), dtype=torch.uint8,
                         device=dev)
        wss = torch.empty(mq.shared_expert_w8a8_rot_workspace_bytes(T, H, Is),
                          dtype=torch.uint8, device=dev)
        wsl = torch.empty(mq.lib().moe_w8a8_rot_shared_workspace_bytes(T, H, E, I, k, Is),
                          dtype=torch.uint8, device=dev)
        sets = []
        ih = hashlib.sha256()
        for r in range(nsets):
            key = (*c["xkey"], 7) if r == 0 else (*c["xkey"], 7, r)
            xh = synth.activations(key, T, H, 0, 1.0)
            ih.update(memoryview(xh).cast("B"))
            sets.append(dict(x=bf16_dev(xh),
                             logits=torch.empty((T, E), dtype=torch.float32, device=dev),
                             ids=torch.empty((T, k), dtype=torch.int32, device=dev),
                             wt=torch.empty((T, k), dtype=torch.float32, device=dev),
                             y=torch.empty((T, H), dtype=torch.float32, device=dev),
                             out=torch.empty((T, H), dtype=torch.bfloat16, device=dev)))
        hashes[f"rot_moe_T{T}_inputs"] = ih.hexdigest()

        def router(i):
            st = sets[i % nsets]
            mq.router_gate_bf16(st["x"], wg, logits=st["logits"])

        def shared(i):
            st = sets[i % nsets]
            mq.shared_expert_w8a8_rot(st["x"], *shared_w, y=st["y"], ws=wss)

        def routed(i):
            st = sets[i % nsets]
            a13, b13, a2, b2 = copies[i % len(copies)]
            mq.moe_w8a8_rot_forward(st["x"], st["logits"], a13, b13, a2, b2, k,
                                    shared=st["y"], topk_ids=st["ids"], topk_w=st["wt"],
                                    out=st["out"], ws=ws)

        def layer(i):
            router(i)
            shared(i)
            routed(i)

        def layer_one_call(i):  # router, then the routed layer with its shared expert
            router(i)
            st = sets[i % nsets]
            a13, b13, a2, b2 = copies[i % len(copies)]
            mq.moe_w8a8_rot_shared_forward(st["x"], st["logits"], a13, b13, a2, b2, k,
                                           shared_w=shared_w, topk_ids=st["ids"],
                                           topk_w=st["wt"], out=st["out"], ws=wsl)

        for r in range(nsets):  # every set through the layer once (untimed)
            layer(r)
        torch.cuda.synchronize()
        touched = sum(int(torch.unique(st["ids"]).numel()) for st in sets) / nsets
        io = T * H * 2 + T * H * 2
        parts = {"router": (router, router_bytes + T * H * 2 + T * E * 4),
                 "shared": (shared, shared_bytes + T * H * 2 + T * H * 4),
                 "routed": (routed, touched * expert_bytes + io + T * H * 4 + T * E * 4),
                 "layer": (layer, touched * expert_bytes + shared_bytes + router_bytes + io),
                 "layer_one_call": (layer_one_call,
                                    touched * expert_bytes + shared_bytes + router_bytes + io)}
        for name, (fn, nbytes) in parts.items():
            _, each = timer.run(fn, it, groups=min(it, 8))
            t = pct(each, 50)
            r = {**timer.stats_us(each), "alg_bytes": int(nbytes),
                 "gbs": round(nbytes / (t * 1e-3) / 1e9, 1),
                 "frac_hbm": round(nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            if name in ("routed", "layer", "layer_one_call"):
                r["tokens_per_s"] = round(T / (t * 1e-3), 1)
                r["experts_touched"] = round(touched, 1)
            res[f"rot_moe_T{T}_{name}"] = r
    del copies
    torch.cuda.empty_cache()
    return res


def hadamard_cases(torch, np, mq, synth, dev, timer, bf16_dev, hashes):
    cfg = synth.hadamard_linear(1)
    K, N = cfg["K"], cfg["N"]
    Wh = synth.weights(cfg["wkey"], N, K)
    hashes["hadamard_weights_fp32"] = sha256_arrays(Wh)
    qw, su8, s2 = mq.fwht128_weight_prep_g256(torch.from_numpy(Wh).to(dev))
    qw = mq.pack_weights(qw)  # MFMA tile layout, untimed
    wbytes = N * K + N * K // 256 + 2 * N
    ncopy = max(2, math.ceil(2 * MALL_BYTES / wbytes) + 1)
    copies = [(qw, su8, s2)] + [(qw.clone(), su8.clone(), s2.clone()) for _ in range(ncopy - 1)]
    res = {}
    for M in (1, 256):
        c = synth.hadamard_linear(M)
        xh = synth.activations(c["xkey"], M, K, c["n_outliers"], c["outlier_scale"],
                               heavy_tail=True)
        hashes[f"hadamard_M{M}_activations"] = sha256_arrays(xh)
        x = bf16_dev(xh)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(mq.linear_w8a8_g256_workspace_bytes(M, N, K), 256),
                         dtype=torch.uint8, device=dev)

        def fn(i):
            w = copies[i % len(copies)]
            mq.linear_w8a8_g256_packed(x, w[0], w[1], w[2], y=y, ws=ws)

        for i in range(3):
            fn(i)
        _, each = timer.run(fn, 64, groups=8)
        t = pct(each, 50)
        nbytes = wbytes + M * K * 2 + 2 * M * N
        res[f"fwht128_g256_M{M}_K{K}_N{N}"] = {
            **timer.stats_us(each),
            "gbs": round(nbytes / (t * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "tops": round(2.0 * M * N * K / (t * 1e-3) / 1e12, 2),
            "weight_copies": len(copies),
        }
    return res


def mlp_cases(torch, np, mq, synth, dev, timer, bf16_dev, hashes):
    """The dense MLP block at the decode and prefill shapes: gate_up K=5120 ->
    2 x 8704 interleaved rows, SiLU(gate)*up, requant, down 8704 -> 5120.
    Decode (M in {1, 2, 4, 8}) is graded on HBM (weights + scales +
    activations in + bf16 out), prefill (M=4096) on int8 MFMA (2 x the MACs
    of both GEMMs).  Weights rotate over copies as in the decode step."""
    K, I, N = 5120, 8704, 5120
    key = (97, 0)
    wgu_h = synth.weights(key, 2 * I, K)
    wd_h = synth.weights(key, N, I, tensor_id=synth.T_W2)
    hashes["mlp_weights_fp32"] = sha256_arrays(wgu_h, wd_h)
    qgu, sgu = mq.quant_per_token_i8(torch.from_numpy(wgu_h).to(dev))
    qd, sd = mq.quant_per_token_i8(torch.from_numpy(wd_h).to(dev))
    del wgu_h, wd_h
    qgu, qd = mq.pack_weights(qgu), mq.pack_weights(qd)
    wbytes = 2 * I * K + 8 * I + N * I + 4 * N
    ncopy = max(2, math.ceil(2 * MALL_BYTES / wbytes) + 1)
    copies = [(qgu, sgu, qd, sd)] + [tuple(t.clone() for t in (qgu, sgu, qd, sd))
                                     for _ in range(ncopy - 1)]
    res = {}
    for M in (1, 2, 4, 8, 4096):
        xh = synth.activations((97, M), M, K, int(round(0.01 * K)) if M <= 8 else 4,
                               10.0 if M <= 8 else 20.0)
        hashes[f"mlp_M{M}_activations"] = sha256_arrays(xh)
        x = bf16_dev(xh)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(mq.mlp_w8a8_workspace_bytes(M, K, I, N), dtype=torch.uint8, device=dev)

        def fn(i):
            a, b, c, d = copies[i % ncopy]
            mq.mlp_w8a8_packed(x, a, b, c, d, I, N, y=y, ws=ws)

        for i in range(3):
            fn(i)
        _, each = timer.run(fn, 10 if M > 8 else 40, groups=10 if M > 8 else 8)
        t = pct(each, 50)
        ops = 2.0 * M * (2 * I * K + N * I)
        nbytes = wbytes + 2 * M * K + 2 * M * N
        r = {**timer.stats_us(each), "tops": round(ops / (t * 1e-3) / 1e12, 2),
             "gbs": round(nbytes / (t * 1e-3) / 1e9, 1), "weight_copies": ncopy}
        if M <= 8:
            r["frac_hbm"] = round(nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        else:
            r["frac_mfma"] = round(ops / (t * 1e-3) / 1e12 / I8_PEAK_TOPS, 4)
        res[f"mlp_M{M}_K{K}_I{I}_N{N}"] = r
    del copies
    torch.cuda.empty_cache()
    return res


def kv_cases(torch, np, mq, synth, dev, timer, bf16_dev, hashes):
    """int8 KV-cache quant with an f16 scale per token and head: 4 KV heads of
    256 (the 27B model's full-attention layers), one decode step of 1 and 8
    sequences and a 4096-token prefill chunk, written through a slot
    mapping into a 32768-row cache.  HBM-graded: bf16 in, int8 codes and f16
    scales out, int32 slots."""
    Hk, D, rows = 4, 256, 32768
    q_cache = torch.zeros((rows, Hk, D), dtype=torch.int8, device=dev)
    s_cache = torch.zeros((rows, Hk), dtype=torch.float16, device=dev)
    res = {}
    for T in (1, 8, 4096):
        xh = synth.activations((100, T), T, Hk * D, int(round(0.01 * Hk * D)), 10.0)
        hashes[f"kv_T{T}"] = sha256_arrays(xh)
        x = bf16_dev(xh).view(T, Hk, D)
        slots = torch.from_numpy(
            np.random.default_rng(T).permutation(rows)[:T].astype(np.int32)).to(dev)
        for i in range(3):
            mq.kv_quant_i8(x, q_cache, s_cache, slots=slots)
        _, each = timer.run(lambda i: mq.kv_quant_i8(x, q_cache, s_cache, slots=slots), 64,
                            groups=8)
        t = pct(each, 50)
        nbytes = T * Hk * D * 2 + T * Hk * D + T * Hk * 2 + 4 * T
        res[f"kv_quant_T{T}_H{Hk}_D{D}"] = {
            **timer.stats_us(each), "gbs": round(nbytes / (t * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return res


def cpu_baseline(np, synth, seconds: float, step_bytes: int):
    """The CPU oracle on the same decode step, on all the host's threads and on
    one thread (each repeated for about `seconds`)."""
    import oracle

    work = []
    for si, (K, N, name) in enumerate(synth.DECODE_SHAPES):
        W = synth.weights(synth.decode_linear(1, si)["wkey"], N, K)
        qw, sw = oracle.quant_rows(W)
        del W
        for M in synth.DECODE_M:
            cfg = synth.decode_linear(M, si)
            x = synth.activations(cfg["xkey"], M, K, cfg["n_outliers"], cfg["outlier_scale"])
            work.append((x, qw, sw))

    def timed(limit):
        reps, t0 = 0, time.perf_counter()
        while True:
            for x, qw, sw in work:
                oracle.linear_w8a8(x, qw, sw)
            reps += 1
            el = time.perf_counter() - t0
            if el >= limit or reps >= 200:
                return reps, el

    all_threads = oracle.threads()
    reps, el = timed(seconds)
    per_step = el / reps
    oracle.set_threads(1)
    reps1, el1 = timed(seconds)
    oracle.set_threads(all_threads)
    per1 = el1 / reps1
    return {"value": round(step_bytes / per_step / 1e9, 3), "unit": "GB/s",
            "cores": all_threads, "kind": "oracle",
            "sample": f"the full decode step (8 linears), {reps} repetitions, "
                      f"{el:.1f} s of CPU work; {per_step * 1e3:.1f} ms per step",
            "single_thread": {"value": round(step_bytes / per1 / 1e9, 3), "unit": "GB/s",
                              "cores": 1, "sample": f"{reps1} repetitions, {el1:.1f} s; "
                                                    f"{per1 * 1e3:.1f} ms per step"},
            "host_cpu": _cpu_model(), "nproc": os.cpu_count()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
