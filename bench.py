#!/usr/bin/env python3
"""Benchmark of the online INT8 W8A8 hot path on one MI355X.

One step = the decode-shaped dense W8A8 workload: for every M in {1, 2, 4, 8}
the gate_up (K=5120, N=17408) and down (K=8704, N=5120) linears, each as
per-token int8 quant of the bf16 activations followed by the int8 GEMM with
the fp32 epilogue to bf16, through linear_w8a8_packed (weights pre-packed at
load; one or two tokens on the down projection run both in one launch).
The roofline figure of the dominant kernel (the decode GEMM) comes from a
pass of the same eight GEMMs on prepared codes, bracketed by HIP events.  Weights
rotate over enough copies that every launch reads them from HBM, not from the
256 MB Infinity Cache.  `value` is the step's algorithmic bytes over its time
(GB/s).

Extra cases on the same JSON line (``cases``): prefill M=4096 TOPS, the
routed MoE layer tokens/s at T in {1, 64, 2048}, and the Hadamard-domain
linear at M in {1, 256}, each with its fraction of the relevant roofline.
Prefill and Hadamard weights rotate over copies as above; the MoE cases
rotate over seeded routing inputs and alternate two copies of the layer's
weights, so consecutive calls read different experts or another copy.

Timing: the stream is first parked on a short spin kernel while the host
enqueues the timed launches, so HIP events measure GPU time rather than
Python launch overhead.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W8A8 GEMM TOPS + HBM GB/s (M=1 & M=4096, % roofline); MoE tokens/s"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
I8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA (5.0 POPS)
MALL_BYTES = 256 << 20     # Infinity Cache
PROBE_ELEMS = 1 << 28      # --probe-copy: 1 GiB of fp32 read and 1 GiB written
DECODE_KERNEL = "k_gemm_skinny"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--cases", default="all", choices=["all", "decode", "none"],
                   help="extra cases on the JSON line")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--probe-copy", action="store_true",
                   help="counter runs: time only the decode GEMM pass (no step, value "
                        "null), then a 1 GiB fp32 negation (reads 1 GiB, writes 1 GiB): the "
                        "reference kernel that scales the HBM byte counters")
    p.add_argument("--traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no benchmark: turn two rocprofv3 --pmc runs of this script "
                        "(FETCH_SIZE, then WRITE_SIZE, with --probe-copy) into "
                        "profiles/traffic_decode_gemm.json")
    return p.parse_args()


def src_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "moe_quant_token_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class GpuTimer:
    """Event timing with the stream parked behind a spin kernel while the host enqueues."""

    def __init__(self, torch):
        self.torch = torch
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

    def run(self, fn, iters: int, park_ms: float = 100.0, marks=None):
        """Run fn(i) for i < iters; returns GPU ms from first to last launch."""
        torch = self.torch
        torch.cuda.synchronize()
        self.park(park_ms)
        t0 = time.perf_counter()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for i in range(iters):
            fn(i)
        e.record()
        if (time.perf_counter() - t0) * 1e3 > park_ms:
            self.enqueue_bound = True
        torch.cuda.synchronize()
        return s.elapsed_time(e)


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


def traffic_from_counters(fetch_dir: str, write_dir: str) -> None:
    """HBM bytes per decode GEMM launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch).

    Each counter is scaled by what it reads for the probe kernel, a plain fp32
    negation over 1 GiB (1 GiB fetched, 1 GiB written), so the figure is in
    bytes of the same kind as the algorithmic ones."""
    out = {"kernel": DECODE_KERNEL, "src_hash": src_hash("gemm_skinny.hip")}
    total = 0.0
    for key, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _counter_rows(d, counter)
        probe = [v for n, v in rows if "neg" in n]
        gemm = [v for n, v in rows if DECODE_KERNEL in n]
        if not probe or not gemm:
            raise SystemExit(f"{counter}: probe dispatches {len(probe)}, gemm dispatches {len(gemm)}")
        scale = float(PROBE_ELEMS * 4) / (max(probe) * 1024.0)
        per = sum(gemm) / len(gemm) * 1024.0 * scale
        out[key] = {"counter": counter, "dispatches": len(gemm), "raw_kib_avg": sum(gemm) / len(gemm),
                    "probe_kib": max(probe), "scale": scale, "bytes_per_launch": per}
        total += per
    out["bytes_per_launch"] = total
    path = os.path.join(ROOT, "profiles", "traffic_decode_gemm.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def main():
    args = parse()
    if args.traffic:
        traffic_from_counters(*args.traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the "
              "kernels run on one GPU's share of a layer; nothing here spans GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_quant_token_amd as mq
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    timer = GpuTimer(torch)

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).to(dev)

    # ------------------------------------------------------------ decode step
    shapes = []
    for si, (K, N, name) in enumerate(synth.DECODE_SHAPES):
        W = torch.from_numpy(synth.weights(synth.decode_linear(1, si)["wkey"], N, K)).to(dev)
        qw, sw = mq.quant_per_token_i8(W)          # weight preparation, untimed
        del W
        qw = mq.pack_weights(qw)                   # MFMA tile layout, untimed
        wbytes = N * K + 4 * N
        ncopy = max(2, math.ceil(2 * MALL_BYTES / wbytes) + 1)
        copies = [(qw, sw)] + [(qw.clone(), sw.clone()) for _ in range(ncopy - 1)]
        shapes.append(dict(K=K, N=N, name=name, copies=copies))
    calls = []
    for M in synth.DECODE_M:
        for si, sh in enumerate(shapes):
            cfg = synth.decode_linear(M, si)
            x = bf16_dev(synth.activations(cfg["xkey"], M, sh["K"], cfg["n_outliers"],
                                           cfg["outlier_scale"]))
            q, s = mq.quant_per_token_i8(x)  # codes for the GEMM-only pass, untimed
            y = torch.empty((M, sh["N"]), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(mq.linear_w8a8_workspace_bytes(M, sh["N"], sh["K"]),
                             dtype=torch.uint8, device=dev)
            calls.append(dict(M=M, sh=sh, x=x, q=q, s=s, y=y, ws=ws, use=0))
    step_bytes = sum(linear_bytes(c["M"], c["sh"]["N"], c["sh"]["K"], True) for c in calls)
    gemm_bytes = sum(linear_bytes(c["M"], c["sh"]["N"], c["sh"]["K"], False) for c in calls)

    L = mq.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream
    ev_pairs = []

    def weights(c):
        sh = c["sh"]
        qw, sw = sh["copies"][c["use"] % len(sh["copies"])]
        c["use"] += 1
        return qw, sw

    def step(i):
        # one decode step: the linear entry point on each of the eight linears
        # (quant + GEMM, or both in one launch where the library does that)
        for c in calls:
            sh = c["sh"]
            qw, sw = weights(c)
            st = L.linear_w8a8_packed(c["x"].data_ptr(), c["M"], sh["K"], sh["K"],
                                      qw.data_ptr(), sw.data_ptr(), sh["N"],
                                      c["y"].data_ptr(), sh["N"], c["ws"].data_ptr(),
                                      c["ws"].numel(), stream)
            if st != 0:
                raise RuntimeError(f"linear_w8a8_packed failed: {st}")

    def gemm_pass(i):
        # the dominant kernel alone: the eight decode GEMMs on prepared codes,
        # bracketed by events on the launch stream
        ea = torch.cuda.Event(enable_timing=True)
        eb = torch.cuda.Event(enable_timing=True)
        ea.record()
        for c in calls:
            sh = c["sh"]
            qw, sw = weights(c)
            st = L.gemm_w8a8_packed(c["q"].data_ptr(), c["s"].data_ptr(), c["M"], sh["K"],
                                    sh["K"], qw.data_ptr(), sw.data_ptr(), sh["N"],
                                    c["y"].data_ptr(), sh["N"], None, 0, stream)
            if st != 0:
                raise RuntimeError(f"gemm_w8a8_packed failed: {st}")
        eb.record()
        ev_pairs.append((ea, eb))

    # the counter runs (--probe-copy) take the GEMM pass only, so every
    # dispatch of the decode GEMM they count is one of the eight shapes
    counters_only = args.probe_copy
    for i in range(args.warmup):
        if not counters_only:
            step(i)
        gemm_pass(i)
    torch.cuda.synchronize()
    ev_pairs.clear()
    total_ms = None if counters_only else timer.run(step, args.steps)
    timer.run(gemm_pass, args.steps)
    gemm_ms = sum(a.elapsed_time(b) for a, b in ev_pairs)
    n_gemm = len(calls) * args.steps
    ms_per_step = None if counters_only else total_ms / args.steps
    value = None if counters_only else step_bytes / (ms_per_step * 1e-3) / 1e9
    gemm_avg_us = gemm_ms * 1e3 / n_gemm
    achieved = (gemm_bytes / len(calls)) / (gemm_avg_us * 1e-6) / 1e9

    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic_decode_gemm.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            tj = json.load(f)
        if tj.get("src_hash") == src_hash("gemm_skinny.hip"):
            traffic = tj.get("bytes_per_launch")

    out = {
        "metric": METRIC,
        "value": None if value is None else round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": None if ms_per_step is None else round(ms_per_step, 5),
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
        "roofline": {
            "kernel": "k_gemm_skinny (decode weight-streaming int8 GEMM)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(gemm_avg_us, 3),
            "bytes_per_launch": gemm_bytes / len(calls),
        },
    }

    # ------------------------------------------------------------ extra cases
    cases = {}
    if args.cases == "all":
        cases.update(prefill_cases(torch, np, mq, synth, dev, timer, bf16_dev))
        cases.update(moe_cases(torch, np, mq, synth, dev, timer, bf16_dev))
        cases.update(hadamard_cases(torch, np, mq, synth, dev, timer, bf16_dev))
    if cases:
        out["cases"] = cases
    if timer.enqueue_bound:
        out["enqueue_bound_warning"] = True

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


def prefill_cases(torch, np, mq, synth, dev, timer, bf16_dev):
    res = {}
    for N in (5120, 17408):
        cfg = synth.prefill_linear(N)
        M, K = cfg["M"], cfg["K"]
        W = torch.from_numpy(synth.weights(cfg["wkey"], N, K)).to(dev)
        qw, sw = mq.quant_per_token_i8(W)
        del W
        qw = mq.pack_weights(qw)
        # weight copies rotate so each launch reads its weights from HBM, not
        # from the Infinity Cache
        ncopy = max(2, math.ceil(2 * MALL_BYTES / (N * K)) + 1)
        copies = [(qw, sw)] + [(qw.clone(), sw.clone()) for _ in range(ncopy - 1)]
        x = bf16_dev(synth.activations(cfg["xkey"], M, K, cfg["n_outliers"],
                                       cfg["outlier_scale"]))
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

        t_g = timer.run(gemm, it) / it
        t_l = timer.run(linear, it) / it
        ops = 2.0 * M * N * K
        res[f"prefill_M{M}_K{K}_N{N}"] = {
            "gemm_us": round(t_g * 1e3, 2),
            "gemm_tops": round(ops / (t_g * 1e-3) / 1e12, 1),
            "gemm_frac_mfma": round(ops / (t_g * 1e-3) / 1e12 / I8_PEAK_TOPS, 4),
            "linear_bf16_us": round(t_l * 1e3, 2),
            "linear_bf16_tops": round(ops / (t_l * 1e-3) / 1e12, 1),
            "linear_frac_mfma": round(ops / (t_l * 1e-3) / 1e12 / I8_PEAK_TOPS, 4),
            "weight_copies": ncopy,
        }
        del qw, sw, x, q, s, y, ws, ws_g, copies
        torch.cuda.empty_cache()
    return res


def moe_cases(torch, np, mq, synth, dev, timer, bf16_dev):
    cfg = synth.moe(1)
    E, H, I, k = cfg["E"], cfg["H"], cfg["I"], cfg["k"]
    w13 = torch.empty((E, 2 * I, H), dtype=torch.int8, device=dev)
    s13 = torch.empty((E, 2 * I), dtype=torch.float32, device=dev)
    w2 = torch.empty((E, H, I), dtype=torch.int8, device=dev)
    s2 = torch.empty((E, H), dtype=torch.float32, device=dev)
    for e in range(E):  # weight preparation on the GPU (untimed)
        a = torch.from_numpy(synth.expert_weights(cfg["wkey"], e, 2 * I, H, synth.T_W)).to(dev)
        mq.quant_per_token_i8(a, q=w13[e], s=s13[e])
        b = torch.from_numpy(synth.expert_weights(cfg["wkey"], e, H, I, synth.T_W2)).to(dev)
        mq.quant_per_token_i8(b, q=w2[e], s=s2[e])
    w13, w2 = mq.pack_moe_weights(w13, w2)  # MFMA tile layout, untimed
    # two copies of the layer's weights, used alternately, and routing inputs
    # rotating over seeded sets: a call reuses an expert's weights only after
    # far more than the 256 MB Infinity Cache has streamed by (at T=1 a call
    # touches 8 experts, 25 MB; the larger batches 700-800 MB per call, most
    # of the experts, which without a second copy the next call would partly
    # find in the cache)
    copies = [(w13, s13, w2, s2), (w13.clone(), s13.clone(), w2.clone(), s2.clone())]
    res = {}
    for T, nsets, it in ((1, 64, 64), (64, 4, 20), (2048, 2, 10)):
        c = synth.moe(T)
        ws = torch.empty(mq.moe_w8a8_workspace_bytes(T, H, E, I, k), dtype=torch.uint8,
                         device=dev)
        sets = []
        for r in range(nsets):
            key = c["xkey"] if r == 0 else (*c["xkey"], r)
            x = bf16_dev(synth.activations(key, T, H, 0, 1.0))
            logits = torch.from_numpy(synth.router_logits(key, T, E)).to(dev)
            ids = torch.empty((T, k), dtype=torch.int32, device=dev)
            wt = torch.empty((T, k), dtype=torch.float32, device=dev)
            out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            sets.append((x, logits, ids, wt, out))

        def fn(i):
            x, logits, ids, wt, out = sets[i % nsets]
            a13, b13, a2, b2 = copies[i % len(copies)]
            mq.moe_w8a8_forward(x, logits, a13, b13, a2, b2, k, topk_ids=ids, topk_w=wt,
                                out=out, ws=ws, packed=True)

        for r in range(nsets):  # every set routed once (ids filled), untimed
            fn(r)
        t = timer.run(fn, it) / it
        touched = sum(int(torch.unique(st[2]).numel()) for st in sets) / nsets
        nbytes = touched * (2 * I * H + H * I + 4 * (2 * I + H)) + T * H * 2 + T * E * 4 + \
            T * H * 2
        ops = 2.0 * T * k * (2 * I * H + H * I)
        res[f"moe_T{T}"] = {
            "us": round(t * 1e3, 2),
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


def hadamard_cases(torch, np, mq, synth, dev, timer, bf16_dev):
    cfg = synth.hadamard_linear(1)
    K, N = cfg["K"], cfg["N"]
    W = torch.from_numpy(synth.weights(cfg["wkey"], N, K)).to(dev)
    qw, su8, s2 = mq.fwht128_weight_prep_g256(W)
    qw = mq.pack_weights(qw)  # MFMA tile layout, untimed
    del W
    wbytes = N * K + N * K // 256 + 2 * N
    ncopy = max(2, math.ceil(2 * MALL_BYTES / wbytes) + 1)
    copies = [(qw, su8, s2)] + [(qw.clone(), su8.clone(), s2.clone()) for _ in range(ncopy - 1)]
    res = {}
    for M in (1, 256):
        c = synth.hadamard_linear(M)
        x = bf16_dev(synth.activations(c["xkey"], M, K, c["n_outliers"], c["outlier_scale"],
                                       heavy_tail=True))
        q = torch.empty((M, K), dtype=torch.int8, device=dev)
        s = torch.empty((M,), dtype=torch.float32, device=dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

        ws = torch.empty(max(mq.linear_w8a8_g256_workspace_bytes(M, N, K), 256),
                         dtype=torch.uint8, device=dev)

        def fn(i):
            w = copies[i % len(copies)]
            mq.linear_w8a8_g256_packed(x, w[0], w[1], w[2], y=y, ws=ws)

        for i in range(3):
            fn(i)
        it = 64
        t = timer.run(fn, it) / it
        nbytes = wbytes + M * K * 2 + 2 * M * N
        res[f"fwht128_g256_M{M}_K{K}_N{N}"] = {
            "us": round(t * 1e3, 2),
            "gbs": round(nbytes / (t * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "tops": round(2.0 * M * N * K / (t * 1e-3) / 1e12, 2),
            "weight_copies": len(copies),
        }
    return res


def cpu_baseline(np, synth, seconds: float, step_bytes: int):
    """The CPU oracle on the same decode step (repeated for about `seconds`)."""
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
    reps = 0
    t0 = time.perf_counter()
    while True:
        for x, qw, sw in work:
            oracle.linear_w8a8(x, qw, sw)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 200:
            break
    per_step = el / reps
    return {"value": round(step_bytes / per_step / 1e9, 3), "unit": "GB/s",
            "cores": oracle.threads(), "kind": "oracle",
            "sample": f"the full decode step (8 linears), {reps} repetitions, "
                      f"{el:.1f} s of CPU work; {per_step * 1e3:.1f} ms per step",
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
