#!/usr/bin/env python3
"""Benchmark of the fused Conv2D -> BatchNorm -> ReLU operator on one MI355X.

One step = one cbr_forward_train call (conv + channel statistics, finalize, normalise +
ReLU + mask) on the headline workload: N=256, 56x56, 64 -> 64 channels, 3x3, stride 1,
pad 1, bf16 NHWC, inputs resident in HBM.  The timed region is exactly --steps calls,
bracketed by device synchronisation; per-kernel durations come from HIP events the
library records on its stream inside the same region.

Printed: one JSON line with the step throughput (TFLOP/s of the convolution, plus
algorithmic HBM GB/s), the roofline of the dominant kernel, the other calls' kernels
(inference and backward workloads, unless --no-aux), and the fp64 CPU oracle timed on
the host as a reported baseline (unless --no-cpu-baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
BF16 = 2


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def conv_flops(g):
    """2 * M * K * R * S * C: multiply-adds of the convolution only."""
    return 2.0 * g.m * g.k * g.r * g.s * g.c


def train_bytes(g):
    """Algorithmic HBM bytes of the fused training forward, per kernel.
    conv: read x and w, write z; apply: read z, write y and the packed mask."""
    x = g.n * g.h * g.w * g.c * BF16
    w = g.k * g.r * g.s * g.c * BF16
    z = g.m * g.k * BF16
    mask = (g.m * g.k + 31) // 32 * 4
    return {"conv_fprop_stats": x + w + z, "bn_stats_finalize": 0, "bn_apply_relu_mask": z + z + mask}


def unfused_train_bytes(g):
    """Three-kernel baseline: conv writes z; BN reads z for statistics, reads it again
    and writes its output; ReLU reads that and writes y plus a one-byte-per-element mask."""
    x = g.n * g.h * g.w * g.c * BF16
    w = g.k * g.r * g.s * g.c * BF16
    z = g.m * g.k * BF16
    return x + w + z + (z + z + z) + (z + z + g.m * g.k)


def infer_bytes(g):
    x = g.n * g.h * g.w * g.c * BF16
    w = g.k * g.r * g.s * g.c * BF16
    y = g.m * g.k * BF16
    return {"bn_fold": w + w, "conv_fprop_bias_relu": x + w + y}


def bwd_bytes(g):
    x = g.n * g.h * g.w * g.c * BF16
    w = g.k * g.r * g.s * g.c * BF16
    z = g.m * g.k * BF16
    mask = (g.m * g.k + 31) // 32 * 4
    dw = g.k * g.r * g.s * g.c * 4
    # BN backward: reduce reads dy, mask, z; apply reads them again and writes dz.
    return {"bn_backward": (z + mask + z) * 2 + z, "conv_wgrad": z + x + dw, "conv_dgrad": z + w + x}


def kernel_entry(name, ms, nbytes, flops, prof=None):
    """Timing of one stage against its algorithmic bytes and flops; prof = (workload,
    kernel-name prefixes) names the stage's kernels in the committed counter summary,
    whose measured HBM bytes per call are added while the library's sources are the ones
    the counters were taken on."""
    t = ms * 1e-3
    gbs = nbytes / t / 1e9 if t > 0 else 0.0
    tfl = flops / t / 1e12 if t > 0 else 0.0
    e = {"kernel": name, "ms": round(ms, 5), "gbps": round(gbs, 1), "tflops": round(tfl, 2),
         "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "mfma_frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4),
         "bytes": int(nbytes), "flops": int(flops)}
    if prof is not None:
        c = counted_stage(*prof)
        if c is not None:
            e["traffic"] = c["traffic"]
            e["traffic_over_algorithmic"] = round(c["traffic"] / nbytes, 3) if nbytes else None
            if c["mfma_util_pct"] is not None:
                e["mfma_util_pct_counter"] = c["mfma_util_pct"]
    return e


COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_bench_workloads.json")
_counters = None


def counted_stage(workload, prefixes):
    """Measured HBM bytes (calibrated FETCH_SIZE + WRITE_SIZE) per call of a stage: the sum
    over the workload's kernels whose names start with one of prefixes and that ran once
    per call (the profiled run makes 5 calls); also the MFMA utilisation of its busiest
    kernel.  None when the summary is missing or was taken on other library sources."""
    global _counters
    if _counters is None:
        try:
            with open(COUNTERS_FILE) as f:
                _counters = json.load(f)
        except (OSError, ValueError):
            _counters = {}
        from conv2d_batchnorm_relu_amd.profile_summary import sources_sha256
        if _counters.get("sources_sha256") != sources_sha256():
            _counters = {}
    rows = [r for r in _counters.get("workloads", {}).get(workload, [])
            if r["kernel"].startswith(tuple(prefixes)) and r["dispatches"] == 5]
    if not rows or any(r["fetch_bytes"] is None or r["write_bytes"] is None for r in rows):
        return None
    util = [r["mfma_util_pct"] for r in rows if r["mfma_util_pct"]]
    return {"traffic": int(sum(r["fetch_bytes"] + r["write_bytes"] for r in rows)),
            "mfma_util_pct": max(util) if util else None}


def roofline_of(entry, traffic=None):
    """The kernel's binding roofline: whichever of HBM bytes and MFMA flops needs more
    time at peak."""
    t_hbm = entry["bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = entry["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if t_mfma > t_hbm:
        return {"kernel": entry["kernel"], "bound": "mfma", "achieved": entry["tflops"],
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": entry["mfma_frac"], "traffic": traffic}
    return {"kernel": entry["kernel"], "bound": "hbm", "achieved": entry["gbps"], "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": entry["hbm_frac"], "traffic": traffic}


def pct(vals, q):
    import numpy as np
    return float(np.percentile(np.asarray(vals), q))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--ramp-s", type=float, default=2.0,
                    help="seconds of untimed headline steps before the warm-up steps: an idle GPU takes "
                         "a second or two of load to reach its steady clocks")
    ap.add_argument("--no-aux", action="store_true", help="skip the inference and backward workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-images", type=int, default=256,
                    help="images of the headline workload the CPU oracle runs (of 256)")
    ap.add_argument("--cold", type=int, default=5, help="steps timed after evicting the caches")
    ap.add_argument("--no-peaks", action="store_true", help="skip the on-box copy and matmul peak runs")
    ap.add_argument("--batch-sweep", default="",
                    help="comma-separated batch sizes <= 256: time the headline layer's conv at each (the "
                         "first images of the headline input) and fit it against the steps per workgroup")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the run, copy this many MiB device-to-device three times (the known-size "
                         "copy that scales HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported here (this operator's "
              "multi-GPU form is data parallelism over the batch; see the sharding notes).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import conv2d_batchnorm_relu_amd as cbr
    from conv2d_batchnorm_relu_amd.inputs import draw_workload, bf16_bits

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_bf16(a):
        return torch.from_numpy(bf16_bits(a).view(np.int16)).to(dev)

    def to_f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

    def shape_of(g):
        return cbr.make_shape(g.n, g.h, g.w, g.c, g.k, g.r, g.s, g.sh, g.ph, stride_w=g.sw, pad_w=g.pw)

    def make_event():
        # torch creates the underlying hipEvent_t on first record; the library then
        # re-records it from its kernels' own dispatch timestamps.
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def timed(fn, nev, steps, warmup):
        """Runs fn warmup times, then `steps` timed calls without events (wall clock,
        bracketed by device synchronisation), then `steps` calls with per-stage kernel
        events; returns (ms per call, [mean ms per stage], [[ms per call] per stage])."""
        for _ in range(warmup):
            fn(None)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn(None)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        evs = [[make_event() for _ in range(nev)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            fn(evs[i])
        torch.cuda.synchronize()
        per = [[evs[i][2 * j].elapsed_time(evs[i][2 * j + 1]) for i in range(steps)] for j in range(nev // 2)]
        stages = [sum(v) / steps for v in per]
        return wall, stages, per

    def spread(vals):
        return {"median": round(pct(vals, 50), 5), "p10": round(pct(vals, 10), 5), "p90": round(pct(vals, 90), 5)}

    # ---------------- headline: training forward ----------------
    log("drawing the headline workload")
    wl, d = draw_workload("s2_train")
    g = wl.geom
    sp = shape_of(g)
    x, w = to_bf16(d["x"]), to_bf16(d["w"])
    gamma, beta = to_f32(d["gamma"]), to_f32(d["beta"])
    rm, rv = to_f32(d["run_mean"]), to_f32(d["run_var"])
    z = torch.empty((g.n, g.p, g.q, g.k), dtype=torch.int16, device=dev)
    y = torch.empty_like(z)
    mask = torch.empty(cbr.cbr_mask_words(sp), dtype=torch.int32, device=dev)
    sm, si = torch.empty(g.k, device=dev), torch.empty(g.k, device=dev)
    rmo, rvo = torch.empty(g.k, device=dev), torch.empty(g.k, device=dev)
    ws = torch.empty(cbr.cbr_workspace_bytes(sp, cbr.CBR_OP_TRAIN), dtype=torch.uint8, device=dev)

    def train_step(events):
        cbr.cbr_forward_train(sp, x, w, gamma, beta, rm, rv, wl.eps, wl.momentum, z, y, mask, sm, si,
                              rmo, rvo, ws, events=events)

    if args.ramp_s > 0:
        log(f"running untimed steps for {args.ramp_s} s (clock ramp)")
        t_end = time.perf_counter() + args.ramp_s
        while time.perf_counter() < t_end:
            for _ in range(20):
                train_step(None)
            torch.cuda.synchronize()
    log(f"timing {args.steps} steps after {args.warmup} warm-up steps")
    ms, stages, per = timed(train_step, 6, args.steps, args.warmup)
    flops = conv_flops(g)
    kb = train_bytes(g)
    kernels = [kernel_entry("conv3x3_c64_stats", stages[0], kb["conv_fprop_stats"], flops,
                            ("train_s2", ["conv3x3_c64_stats"])),
               kernel_entry("bn_stats_finalize", stages[1], 0, 0),
               kernel_entry("bn_apply_relu_mask", stages[2], kb["bn_apply_relu_mask"], 0,
                            ("train_s2", ["bn_apply_relu_mask"]))]
    dominant = max(kernels, key=lambda e: e["ms"])
    total_bytes = sum(kb.values())

    # cold steps: evict the 256 MB last-level cache before each one
    cold = []
    if args.cold > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        for _ in range(args.cold):
            flush.fill_(1)
            ev = [make_event() for _ in range(6)]
            torch.cuda.synchronize()
            train_step(ev)
            torch.cuda.synchronize()
            cold.append(ev[0].elapsed_time(ev[5]))   # first kernel's start to last kernel's end
        del flush
    cold_ms = float(np.median(cold)) if cold else None

    out = {
        "metric": "CBR train-fwd TFLOP/s + HBM GB/s (% roofline), N256 56x56 64->64 3x3 bf16",
        "value": round(flops / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ramp_s": args.ramp_s,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "train forward N256 56x56 C64->K64 3x3 s1 p1 bf16 NHWC",
                   "n": g.n, "h": g.h, "w": g.w, "c": g.c, "k": g.k, "r": g.r, "s": g.s,
                   "stride": g.stride, "pad": g.pad, "seed": wl.seed},
        "gbps": round(total_bytes / (ms * 1e-3) / 1e9, 1),
        "step_roofline_frac": round(total_bytes / (HBM_PEAK_GBS * 1e9) / (ms * 1e-3), 4),
        "bytes_per_step": int(total_bytes),
        "unfused_bytes": int(unfused_train_bytes(g)),
        "roofline": roofline_of(dominant, dominant.get("traffic")),
        "kernels": kernels,
        "kernel_ms_spread": {e["kernel"]: spread(v) for e, v in zip(kernels, per)},
        "cold_ms_per_step": None if cold_ms is None else round(cold_ms, 5),
    }
    if args.batch_sweep:
        # The persistent conv gives each workgroup a contiguous range of 256-pixel steps
        # (13 per 56x56 image); its time is about a fixed part plus a cost per step of the
        # busiest workgroup.
        spi = -(-g.h * g.w // 256)
        rows = []
        lib = cbr._load()
        lib.cbr_set_plan_override(0, 1)   # the persistent conv at every batch size
        for nb in (int(v) for v in args.batch_sweep.split(",")):
            assert 1 <= nb <= g.n, f"--batch-sweep sizes must lie in 1..{g.n}"
            spn = cbr.make_shape(nb, g.h, g.w, g.c, g.k, g.r, g.s, g.sh, g.ph, stride_w=g.sw, pad_w=g.pw)

            def sweep_step(events):
                cbr.cbr_forward_train(spn, x[:nb], w, gamma, beta, rm, rv, wl.eps, wl.momentum, z[:nb], y[:nb],
                                      mask[:cbr.cbr_mask_words(spn)], sm, si, rmo, rvo, ws, events=events)

            msn, stn, pern = timed(sweep_step, 6, 40, 10)
            tot = nb * spi
            rows.append({"n": nb, "max_steps_per_workgroup": -(-tot // min(tot, 256)),
                         "conv_us": round(pct(pern[0], 50) * 1e3, 2), "call_us": round(msn * 1e3, 2)})
            log(f"batch sweep N = {nb}: conv {rows[-1]['conv_us']} us")
        lib.cbr_set_plan_override(0, 0)
        slope, icpt = np.polyfit([r["max_steps_per_workgroup"] for r in rows], [r["conv_us"] for r in rows], 1)
        out["batch_sweep"] = {"workload": "headline layer's conv at batch n (median of 40 calls)", "rows": rows,
                              "fit_conv_us": {"fixed": round(float(icpt), 2), "per_step": round(float(slope), 3)}}

    del z, y, mask, ws, x
    torch.cuda.empty_cache()

    # ---------------- other calls ----------------
    if not args.no_aux:
        aux = {}
        steps = max(10, args.steps // 5)
        log("inference workload")
        wl4, d4 = draw_workload("s3_infer")
        g4 = wl4.geom
        sp4 = shape_of(g4)
        t4 = dict(x=to_bf16(d4["x"]), w=to_bf16(d4["w"]), b=to_f32(d4["bias"]), ga=to_f32(d4["gamma"]),
                  be=to_f32(d4["beta"]), rm=to_f32(d4["run_mean"]), rv=to_f32(d4["run_var"]),
                  y=torch.empty((g4.n, g4.p, g4.q, g4.k), dtype=torch.int16, device=dev),
                  ws=torch.empty(cbr.cbr_workspace_bytes(sp4, cbr.CBR_OP_INFER), dtype=torch.uint8, device=dev))

        def infer_step(events):
            cbr.cbr_forward_infer(sp4, t4["x"], t4["w"], t4["b"], t4["ga"], t4["be"], t4["rm"], t4["rv"],
                                  wl4.eps, t4["y"], t4["ws"], events=events)

        ms4, st4, _ = timed(infer_step, 4, steps, 5)
        ib = infer_bytes(g4)
        aux["infer"] = {"workload": "infer N256 28x28 C128->K128 3x3 s1 p1 (conv bias)", "ms": round(ms4, 5),
                        "tflops": round(conv_flops(g4) / (ms4 * 1e-3) / 1e12, 2),
                        "kernels": [kernel_entry("bn_fold", st4[0], ib["bn_fold"], 0, ("infer_s3", ["bn_fold"])),
                                    kernel_entry("conv_fprop_bias_relu", st4[1], ib["conv_fprop_bias_relu"],
                                                 conv_flops(g4), ("infer_s3", ["conv_igemm", "conv_fprop"]))]}
        log("conv + bias + relu workload")

        def cbr_step(events):
            cbr.cbr_conv2d_bias_relu(sp4, t4["x"], t4["w"], t4["b"], t4["y"], events=events)

        ms4c, st4c, _ = timed(cbr_step, 2, steps, 5)
        aux["conv_bias_relu"] = {"workload": "Conv2D + bias + ReLU, no BN: N256 28x28 C128->K128 3x3 s1 p1",
                                 "ms": round(ms4c, 5), "tflops": round(conv_flops(g4) / (ms4c * 1e-3) / 1e12, 2),
                                 "kernels": [kernel_entry("conv_bias_relu", st4c[0], ib["conv_fprop_bias_relu"],
                                                          conv_flops(g4), ("conv_bias_relu", ["conv_igemm", "conv_fprop"]))]}
        del t4
        log("backward workload")
        wl5, d5 = draw_workload("s4_bwd")
        g5 = wl5.geom
        sp5 = shape_of(g5)
        t5 = dict(x=to_bf16(d5["x"]), w=to_bf16(d5["w"]), ga=to_f32(d5["gamma"]), be=to_f32(d5["beta"]),
                  rm=to_f32(d5["run_mean"]), rv=to_f32(d5["run_var"]), dy=to_bf16(d5["dy"]))
        zz = torch.empty((g5.n, g5.p, g5.q, g5.k), dtype=torch.int16, device=dev)
        yy = torch.empty_like(zz)
        mk = torch.empty(cbr.cbr_mask_words(sp5), dtype=torch.int32, device=dev)
        s5m, s5i = torch.empty(g5.k, device=dev), torch.empty(g5.k, device=dev)
        r5m, r5v = torch.empty(g5.k, device=dev), torch.empty(g5.k, device=dev)
        ws5 = torch.empty(max(cbr.cbr_workspace_bytes(sp5, cbr.CBR_OP_TRAIN),
                              cbr.cbr_workspace_bytes(sp5, cbr.CBR_OP_BWD)), dtype=torch.uint8, device=dev)

        def fwd5(events):
            cbr.cbr_forward_train(sp5, t5["x"], t5["w"], t5["ga"], t5["be"], t5["rm"], t5["rv"], wl5.eps,
                                  wl5.momentum, zz, yy, mk, s5m, s5i, r5m, r5v, ws5, events=events)

        fwd5(None)
        dz = torch.empty_like(zz)
        dgam, dbet = torch.empty(g5.k, device=dev), torch.empty(g5.k, device=dev)
        dw = torch.empty((g5.k, g5.r, g5.s, g5.c), device=dev)
        dx = torch.empty((g5.n, g5.h, g5.w, g5.c), dtype=torch.int16, device=dev)

        def bwd_step(events):
            cbr.cbr_backward(sp5, t5["x"], t5["w"], zz, mk, t5["dy"], t5["ga"], s5m, s5i, dz, dgam, dbet, dw,
                             dx, ws5, events=events)

        ms5, st5, _ = timed(bwd_step, 6, steps, 5)
        bb = bwd_bytes(g5)
        f5 = conv_flops(g5)
        aux["backward"] = {"workload": "backward N256 14x14 C256->K256 3x3 s1 p1", "ms": round(ms5, 5),
                           "tflops": round(2 * f5 / (ms5 * 1e-3) / 1e12, 2),
                           "kernels": [kernel_entry("bn_backward", st5[0], bb["bn_backward"], 0, ("bwd_s4", ["bnbwd_"])),
                                       kernel_entry("conv_wgrad", st5[1], bb["conv_wgrad"], f5,
                                                    ("bwd_s4", ["conv_wgrad", "split_sum"])),
                                       kernel_entry("conv_dgrad", st5[2], bb["conv_dgrad"], f5,
                                                    ("bwd_s4", ["flip_weights", "conv_igemm", "conv_fprop"]))]}
        ms5f, st5f, _ = timed(fwd5, 6, steps, 5)
        aux["train_s4"] = {"workload": "train forward N256 14x14 C256->K256 3x3", "ms": round(ms5f, 5),
                           "tflops": round(f5 / (ms5f * 1e-3) / 1e12, 2)}
        del t5, zz, yy, mk, ws5, dz, dx
        torch.cuda.empty_cache()
        log("first-layer workload")
        wl2, d2 = draw_workload("stem")
        g2 = wl2.geom
        sp2 = shape_of(g2)
        t2 = dict(x=to_bf16(d2["x"]), w=to_bf16(d2["w"]), ga=to_f32(d2["gamma"]), be=to_f32(d2["beta"]),
                  rm=to_f32(d2["run_mean"]), rv=to_f32(d2["run_var"]))
        z2 = torch.empty((g2.n, g2.p, g2.q, g2.k), dtype=torch.int16, device=dev)
        y2 = torch.empty_like(z2)
        m2 = torch.empty(cbr.cbr_mask_words(sp2), dtype=torch.int32, device=dev)
        v2 = [torch.empty(g2.k, device=dev) for _ in range(4)]
        ws2 = torch.empty(cbr.cbr_workspace_bytes(sp2, cbr.CBR_OP_TRAIN), dtype=torch.uint8, device=dev)

        def stem_step(events):
            cbr.cbr_forward_train(sp2, t2["x"], t2["w"], t2["ga"], t2["be"], t2["rm"], t2["rv"], wl2.eps,
                                  wl2.momentum, z2, y2, m2, v2[0], v2[1], v2[2], v2[3], ws2, events=events)

        ms2, st2, _ = timed(stem_step, 6, steps, 5)
        kb2 = train_bytes(g2)
        aux["stem_train"] = {"workload": "train forward N64 224x224 C3->K64 7x7 s2 p3", "ms": round(ms2, 5),
                             "gbps": round(sum(kb2.values()) / (ms2 * 1e-3) / 1e9, 1),
                             "kernels": [kernel_entry("conv_fprop_stats(first layer)", st2[0],
                                                      kb2["conv_fprop_stats"], conv_flops(g2),
                                                      ("train_stem", ["conv_c3s2"])),
                                         kernel_entry("bn_stats_finalize", st2[1], 0, 0),
                                         kernel_entry("bn_apply_relu_mask", st2[2], kb2["bn_apply_relu_mask"], 0,
                                                      ("train_stem", ["bn_apply_relu_mask"]))]}
        del t2, z2, y2, m2, ws2
        # the headline layer at other batch sizes: N = 32 (one GPU's share of 256 over 8)
        # and N = 300 (more images than CUs); the persistent conv forced, as in the tests
        import ctypes
        lib = cbr._load()
        for nb in (32, 300):
            log(f"headline layer at N = {nb}")
            wlb, db = draw_workload("s2_train", n=nb)
            gb = wlb.geom
            spb = shape_of(gb)
            lib.cbr_set_plan_override(0, 1)
            try:
                tb = dict(x=to_bf16(db["x"]), w=to_bf16(db["w"]), ga=to_f32(db["gamma"]), be=to_f32(db["beta"]),
                          rm=to_f32(db["run_mean"]), rv=to_f32(db["run_var"]))
                zb = torch.empty((gb.n, gb.p, gb.q, gb.k), dtype=torch.int16, device=dev)
                yb = torch.empty_like(zb)
                mb = torch.empty(cbr.cbr_mask_words(spb), dtype=torch.int32, device=dev)
                vb = [torch.empty(gb.k, device=dev) for _ in range(4)]
                wsb = torch.empty(cbr.cbr_workspace_bytes(spb, cbr.CBR_OP_TRAIN), dtype=torch.uint8, device=dev)

                def nb_step(events):
                    cbr.cbr_forward_train(spb, tb["x"], tb["w"], tb["ga"], tb["be"], tb["rm"], tb["rv"], wlb.eps,
                                          wlb.momentum, zb, yb, mb, vb[0], vb[1], vb[2], vb[3], wsb, events=events)

                msb, stb, _ = timed(nb_step, 6, steps, 5)
            finally:
                lib.cbr_set_plan_override(0, 0)
            aux[f"train_s2_n{nb}"] = {"workload": f"train forward N{nb} 56x56 C64->K64 3x3 (persistent conv)",
                                      "ms": round(msb, 5), "conv_ms": round(stb[0], 5),
                                      "images_per_ms": round(nb / msb, 2),
                                      "conv_images_per_ms": round(nb / stb[0], 2)}
            del tb, zb, yb, mb, wsb
        out["aux"] = aux

    # ---------------- on-box peaks: streaming copy and a large bf16 matmul ----------------
    if not args.no_peaks:
        log("on-box peaks")
        nb = 1 << 30
        src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(3)
        dst = torch.empty_like(src)
        def ev_time(fn, reps):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ts = []
            for _ in range(reps):
                e0.record(); fn(); e1.record(); torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            return pct(ts, 50)
        t_copy = ev_time(lambda: dst.copy_(src), 10)
        del src, dst
        a = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
        b = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
        t_mm = ev_time(lambda: torch.matmul(a, b), 10)
        del a, b
        copy_gbs = 2 * nb / (t_copy * 1e-3) / 1e9
        mm_tfl = 2 * 8192 ** 3 / (t_mm * 1e-3) / 1e12
        r = out["roofline"]
        box_peak = copy_gbs if r["unit"] == "GB/s" else mm_tfl
        out["onbox_peaks"] = {"copy_gbps": round(copy_gbs, 1), "bf16_matmul_tflops": round(mm_tfl, 1),
                              "copy": "1 GiB device-to-device copy (read + write bytes)",
                              "matmul": "torch.matmul bf16 8192^3 (hipBLASLt)",
                              "dominant_frac_of_onbox_peak": round(r["achieved"] / box_peak, 4)}
        torch.cuda.empty_cache()

    if args.calib_copy_mib > 0:
        nb = args.calib_copy_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(5)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------- CPU baseline: the fp64 oracle on the host ----------------
    if not args.no_cpu_baseline:
        import oracle
        n = max(1, min(args.cpu_images, g.n))
        log(f"CPU oracle on {n} of {g.n} images")
        sub = {k: (v[:n] if k == "x" else v) for k, v in d.items()}
        gs = g.with_n(n)
        osp = oracle.OShape(gs.n, gs.h, gs.w, gs.c, gs.k, gs.r, gs.s, gs.stride, gs.stride, gs.pad, gs.pad)
        t0 = time.perf_counter()
        oracle.forward_train(osp, sub["x"], sub["w"], sub["gamma"], sub["beta"], sub["run_mean"],
                             sub["run_var"], wl.eps, wl.momentum)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(conv_flops(gs) / dt / 1e12, 6), "unit": "TFLOP/s",
                               "cores": oracle.num_threads(), "kind": "oracle",
                               "sample": f"train forward on {n} of {g.n} images of the headline workload "
                                         f"(fp64 direct loops), {dt:.2f} s"}
        # the same oracle on one thread, on a smaller sample
        n1 = max(1, n // 16)
        g1 = g.with_n(n1)
        o1 = oracle.OShape(g1.n, g1.h, g1.w, g1.c, g1.k, g1.r, g1.s, g1.stride, g1.stride, g1.pad, g1.pad)
        nthreads = oracle.num_threads()
        oracle.set_num_threads(1)
        t0 = time.perf_counter()
        oracle.forward_train(o1, sub["x"][:n1], sub["w"], sub["gamma"], sub["beta"], sub["run_mean"],
                             sub["run_var"], wl.eps, wl.momentum)
        dt1 = time.perf_counter() - t0
        oracle.set_num_threads(nthreads)
        out["cpu_baseline_1thread"] = {"value": round(conv_flops(g1) / dt1 / 1e12, 6), "unit": "TFLOP/s",
                                       "cores": 1, "kind": "oracle",
                                       "sample": f"train forward on {n1} of {g.n} images, {dt1:.2f} s"}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
