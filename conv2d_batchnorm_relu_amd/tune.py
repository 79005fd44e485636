"""Offline tuner of the per-shape kernel plans (the MI355X counterpart of the CBR page's
empirical engine search, section 7, and of the TileLang page's autotuned tile
configurations).

For every layer shape of a list (the conv layers of ResNet-50 and VGG16-BN at the given
batch sizes) and every stage of a call -- the training forward's conv, the inference
conv, the data gradient, the weight gradient, the backward's schedule -- it times each plan the library reports
eligible (cbr_plan_eligible), forcing it with cbr_set_plan_override, and keeps the
fastest.  It writes the table that csrc/cbr_plan.cpp compiles in (cbr_tune_table.inc)
and a markdown summary of every timing.  Rebuild the library after replacing the table.

    python -m conv2d_batchnorm_relu_amd.tune --out-dir <out> [--batch 32 256] [--reps 10]
        [--match '56x56 64->64 3x3'] [--stages 0 1]

A stage's plans are compared by the time of the whole call that contains the stage (the
training forward, the conv + bias + ReLU call, the backward), measured with HIP events
around --reps back-to-back calls (median of three such runs, after a warm-up), so the
figure is the GPU's time per call rather than the host's enqueue time.  Inputs are
synthetic N(0,1) tensors (values do not change the kernels' work).
"""
from __future__ import annotations

import argparse
import ctypes
import os
import statistics
import sys
import time

STAGES = {0: "train_conv", 1: "infer_conv", 2: "dgrad", 3: "wgrad", 4: "backward"}


def resnet50_layers():
    """(H, W, C, K, R, S, stride, pad) of ResNet-50's conv layers (v1.5: stride on the 3x3)."""
    L = [(224, 224, 3, 64, 7, 7, 2, 3)]
    for hw, cin, mid, out, first_stride in ((56, 64, 64, 256, 1), (56, 256, 128, 512, 2),
                                             (28, 512, 256, 1024, 2), (14, 1024, 512, 2048, 2)):
        ohw = hw // first_stride
        L += [(hw, hw, cin, mid, 1, 1, 1, 0),                  # first block's 1x1 reduce
              (hw, hw, mid, mid, 3, 3, first_stride, 1),       # first block's 3x3
              (ohw, ohw, mid, out, 1, 1, 1, 0),                # 1x1 expand
              (hw, hw, cin, out, 1, 1, first_stride, 0),       # projection shortcut
              (ohw, ohw, out, mid, 1, 1, 1, 0),                # later blocks' 1x1 reduce
              (ohw, ohw, mid, mid, 3, 3, 1, 1)]                # later blocks' 3x3
    return sorted(set(L), key=L.index)


def vgg16_layers():
    L = []
    for hw, cin, cout, n in ((224, 3, 64, 1), (224, 64, 64, 1), (112, 64, 128, 1), (112, 128, 128, 1),
                             (56, 128, 256, 1), (56, 256, 256, 1), (28, 256, 512, 1), (28, 512, 512, 1),
                             (14, 512, 512, 1)):
        L.append((hw, hw, cin, cout, 3, 3, 1, 1))
    return L


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--out-dir", default="tune_out")
    ap.add_argument("--batch", type=int, nargs="+", default=[32, 256])
    ap.add_argument("--vgg-batch", type=int, nargs="*", default=[32])
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--max-elems", type=int, default=1 << 29, help="skip layers whose tensors exceed this")
    ap.add_argument("--match", default=None,
                    help="only layers whose label 'HxW C->K RxS/stride' contains this text (e.g. '56x56 64->64 3x3')")
    ap.add_argument("--stages", type=int, nargs="+", default=list(STAGES), help="stages to time (0..4)")
    args = ap.parse_args(argv)

    import torch
    import conv2d_batchnorm_relu_amd as cbr

    lib = cbr._load()
    lib.cbr_plan_name.restype = ctypes.c_char_p
    plans = []   # every plan id the library names (ids run from 1 without gaps)
    for p in range(1, 64):
        if lib.cbr_plan_name(p).decode() == "unknown":
            break
        plans.append(p)
    dev = torch.device("cuda:0")
    os.makedirs(args.out_dir, exist_ok=True)

    def log(msg):
        print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)

    layers = [("resnet50", n, L) for n in args.batch for L in resnet50_layers()]
    layers += [("vgg16bn", n, L) for n in args.vgg_batch for L in vgg16_layers()]
    entries, report = [], []
    for net, n, (h, w, c, k, r, s, st, pd) in layers:
        if args.match is not None and args.match not in f"{h}x{w} {c}->{k} {r}x{s}/{st}":
            continue
        sp = cbr.make_shape(n, h, w, c, k, r, s, st, pd)
        try:
            P, Q = cbr.cbr_output_hw(sp)
        except cbr.CbrError as e:
            log(f"skip {net} {n}x{h}x{w}x{c}->{k} {r}x{s}/{st}: {e}")
            continue
        if max(n * h * w * c, n * P * Q * k) > args.max_elems:
            log(f"skip {net} {n}x{h}x{w}x{c}->{k}: larger than --max-elems")
            continue
        x = torch.randn(n, h, w, c, device=dev).to(torch.bfloat16)
        wt = (torch.rand(k, r, s, c, device=dev) - 0.5).to(torch.bfloat16)
        vk = [torch.rand(k, device=dev) + 0.5 for _ in range(6)]
        z = torch.empty(n, P, Q, k, dtype=torch.bfloat16, device=dev)
        y = torch.empty_like(z)
        mask = torch.empty(cbr.cbr_mask_words(sp), dtype=torch.int32, device=dev)
        dy = torch.randn(n, P, Q, k, device=dev).to(torch.bfloat16)
        dz = torch.empty_like(z)
        dwt = torch.empty(k, r, s, c, device=dev)
        dx = torch.empty_like(x) if st == 1 else None

        ws_t = ws_b = None

        def run_train(ev):
            cbr.cbr_forward_train(sp, x, wt, vk[0], vk[1], vk[2], vk[3], 1e-5, 0.1, z, y, mask, vk[4], vk[5],
                                  vk[2], vk[3], ws_t, events=ev)

        def run_infer(ev):
            cbr.cbr_conv2d_bias_relu(sp, x, wt, vk[0], y, events=ev)

        def run_bwd(ev):
            cbr.cbr_backward(sp, x, wt, z, mask, dy, vk[0], vk[4], vk[5], dz, vk[1], vk[2], dwt, dx, ws_b, events=ev)

        def run_bwd_nodz(ev):   # the backward's schedule is compared without a dz output
            cbr.cbr_backward(sp, x, wt, z, mask, dy, vk[0], vk[4], vk[5], None, vk[1], vk[2], dwt, dx, ws_b, events=ev)

        def workspaces():
            t = torch.empty(max(256, cbr.cbr_workspace_bytes(sp, cbr.CBR_OP_TRAIN)), dtype=torch.uint8, device=dev)
            b = torch.empty(max(256, cbr.cbr_workspace_bytes(sp, cbr.CBR_OP_BWD)), dtype=torch.uint8, device=dev)
            return t, b

        ws_t, ws_b = workspaces()
        run_train(None)   # a z, mask and saved statistics for the backward
        torch.cuda.synchronize()
        for stage, sname in STAGES.items():
            if stage not in args.stages:
                continue
            if stage in (2, 4) and st != 1:
                continue   # the data gradient needs stride 1
            cands = [p for p in plans if lib.cbr_plan_eligible(ctypes.byref(sp), stage, p) == 1]
            default = lib.cbr_plan_of(ctypes.byref(sp), stage)
            times = {}
            # a stage's plan is rated by the whole call that contains it, timed over
            # back-to-back calls (the GPU's time per call, not the host's enqueue time)
            fn = run_train if stage == 0 else run_infer if stage == 1 else run_bwd if stage < 4 else run_bwd_nodz
            for plan in cands:
                lib.cbr_set_plan_override(stage, plan)
                try:
                    ws_t, ws_b = workspaces()
                    for _ in range(args.warmup):
                        fn(None)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    ts = []
                    for _ in range(3):
                        torch.cuda.synchronize()
                        e0.record()
                        for _ in range(args.reps):
                            fn(None)
                        e1.record()
                        torch.cuda.synchronize()
                        ts.append(e0.elapsed_time(e1) * 1000.0 / args.reps)
                    times[plan] = statistics.median(ts)
                finally:
                    lib.cbr_set_plan_override(stage, 0)
            if not times:
                continue
            best = min(times, key=times.get)
            name = lambda p: lib.cbr_plan_name(p).decode()
            log(f"{net} N{n} {h}x{w} {c}->{k} {r}x{s}/{st} {sname}: " +
                ", ".join(f"{name(p)} {t:.1f}us" for p, t in sorted(times.items(), key=lambda kv: kv[1])) +
                f" (default {name(default)})")
            report.append((net, n, h, w, c, k, r, s, st, pd, sname, times, best, default))
            if len(times) > 1:
                runner = sorted(times.values())[1]
                entries.append(f"    {{{stage}, {n}, {h}, {w}, {c}, {k}, {r}, {s}, {st}, {st}, {pd}, {pd}, {best}}},"
                               f"   // {net} {sname}: {name(best)} {times[best]:.1f} us, next {runner:.1f} us")
        del x, wt, z, y, mask, dy, dz, dwt, dx, ws_t, ws_b
        torch.cuda.empty_cache()

    inc = os.path.join(args.out_dir, "cbr_tune_table.inc")
    with open(inc, "w") as f:
        f.write("// cbr_tune_table.inc -- per-shape kernel plans measured by the offline tuner\n"
                "// (conv2d_batchnorm_relu_amd/tune.py).  Each entry: the stage, the layer's shape (N, H, W,\n"
                "// C, K, R, S, stride_h, stride_w, pad_h, pad_w) and the plan that ran the stage fastest.\n"
                "// Shapes not listed take the default rule.\n")
        f.write(f"// command: python -m conv2d_batchnorm_relu_amd.tune {' '.join(argv or sys.argv[1:])}\n")
        f.write("\n".join(entries) + "\n")
    md = os.path.join(args.out_dir, "tune_report.md")
    with open(md, "w") as f:
        f.write("| net | N | HxW | C->K | RxS/stride | stage | plans (us, median) | chosen | default |\n")
        f.write("|---|---|---|---|---|---|---|---|---|\n")
        name = lambda p: lib.cbr_plan_name(p).decode()
        for net, n, h, w, c, k, r, s, st, pd, sname, times, best, default in report:
            f.write(f"| {net} | {n} | {h}x{w} | {c}->{k} | {r}x{s}/{st} | {sname} | " +
                    ", ".join(f"{name(p)} {t:.1f}" for p, t in sorted(times.items(), key=lambda kv: kv[1])) +
                    f" | {name(best)} | {name(default)} |\n")
    log(f"wrote {inc} ({len(entries)} entries) and {md}")


if __name__ == "__main__":
    main()
