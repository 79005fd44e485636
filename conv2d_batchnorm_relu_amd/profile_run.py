"""Runs one of the benchmark's workloads a few times, so that rocprofv3 can take per-kernel
counters of that workload alone (one counter pass per run):

    cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/<workload>/fetch -o run -- \\
        python3 -m conv2d_batchnorm_relu_amd.profile_run --workload train_s2 --reps 5

Workloads (the benchmark's shapes and input recipes):
    train_s2        training forward, N256 56x56 C64->K64 3x3 s1 p1
    train_s2_n32    the same layer at N 32 (persistent conv)
    train_s2_n300   the same layer at N 300 (persistent conv)
    infer_s3        folded-BN inference, N256 28x28 C128->K128 3x3 s1 p1
    conv_bias_relu  Conv2D + bias + ReLU without BN on the inference shape
    train_s4        training forward, N256 14x14 C256->K256 3x3 s1 p1 (state for bwd_s4)
    bwd_s4          backward of that layer (dz, dgamma, dbeta, dw, dx)
    train_stem      training forward of the first layer, N64 224x224 C3->K64 7x7 s2 p3
    copy            a 512 MiB device-to-device copy: the calibration kernel of the HBM
                    byte counters (its bytes read and written are known exactly)
"""
from __future__ import annotations

import argparse
import sys

WORKLOAD_NAMES = ("train_s2", "train_s2_n32", "train_s2_n300", "infer_s3", "conv_bias_relu", "train_s4",
                  "bwd_s4", "train_stem", "copy")
COPY_BYTES = 512 << 20


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", required=True, choices=WORKLOAD_NAMES)
    ap.add_argument("--reps", type=int, default=5)
    args = ap.parse_args(argv)

    import torch
    import conv2d_batchnorm_relu_amd as cbr
    from conv2d_batchnorm_relu_amd.inputs import bf16_bits, draw_workload

    dev = torch.device("cuda:0")
    wname = args.workload

    if wname == "copy":
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(5)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.reps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copy: {args.reps} x {COPY_BYTES} bytes", flush=True)
        return 0

    def bf16(a):
        return torch.from_numpy(bf16_bits(a).view("int16")).to(dev)

    def f32(a):
        return torch.from_numpy(a).to(dev)

    base = {"train_s2": ("s2_train", None), "train_s2_n32": ("s2_train", 32), "train_s2_n300": ("s2_train", 300),
            "infer_s3": ("s3_infer", None), "conv_bias_relu": ("s3_infer", None), "train_s4": ("s4_bwd", None),
            "bwd_s4": ("s4_bwd", None), "train_stem": ("stem", None)}[wname]
    wl, d = draw_workload(base[0], n=base[1])
    g = wl.geom
    sp = cbr.make_shape(g.n, g.h, g.w, g.c, g.k, g.r, g.s, g.sh, g.ph, stride_w=g.sw, pad_w=g.pw)
    x, w = bf16(d["x"]), bf16(d["w"])
    out = torch.empty((g.n, g.p, g.q, g.k), dtype=torch.int16, device=dev)

    if wname in ("infer_s3", "conv_bias_relu"):
        b = f32(d["bias"])
        if wname == "infer_s3":
            ws = torch.empty(cbr.cbr_workspace_bytes(sp, cbr.CBR_OP_INFER), dtype=torch.uint8, device=dev)
            vec = [f32(d[k]) for k in ("gamma", "beta", "run_mean", "run_var")]
            call = lambda: cbr.cbr_forward_infer(sp, x, w, b, *vec, wl.eps, out, ws)
        else:
            call = lambda: cbr.cbr_conv2d_bias_relu(sp, x, w, b, out)
    else:
        y = torch.empty_like(out)
        mask = torch.empty(cbr.cbr_mask_words(sp), dtype=torch.int32, device=dev)
        vec = [f32(d[k]) for k in ("gamma", "beta", "run_mean", "run_var")]
        stats = [torch.empty(g.k, device=dev) for _ in range(4)]
        ws = torch.empty(max(cbr.cbr_workspace_bytes(sp, cbr.CBR_OP_TRAIN), cbr.cbr_workspace_bytes(sp, cbr.CBR_OP_BWD)),
                         dtype=torch.uint8, device=dev)
        lib = cbr._load()
        forced = wname in ("train_s2_n32", "train_s2_n300")
        if forced:
            lib.cbr_set_plan_override(0, 1)   # the persistent 3x3 conv
        try:
            train = lambda: cbr.cbr_forward_train(sp, x, w, *vec, wl.eps, wl.momentum, out, y, mask, *stats, ws)
            if wname == "bwd_s4":
                train()
                dy = bf16(d["dy"])
                dz = torch.empty_like(out)
                dgb = [torch.empty(g.k, device=dev) for _ in range(2)]
                dw = torch.empty((g.k, g.r, g.s, g.c), device=dev)
                dx = torch.empty((g.n, g.h, g.w, g.c), dtype=torch.int16, device=dev)
                call = lambda: cbr.cbr_backward(sp, x, w, out, mask, dy, vec[0], stats[0], stats[1], dz, dgb[0],
                                                dgb[1], dw, dx, ws)
            else:
                call = train
            torch.cuda.synchronize()
            for _ in range(args.reps):
                call()
            torch.cuda.synchronize()
        finally:
            if forced:
                lib.cbr_set_plan_override(0, 0)
        print(f"{wname}: {args.reps} calls of {g}", flush=True)
        return 0

    torch.cuda.synchronize()
    for _ in range(args.reps):
        call()
    torch.cuda.synchronize()
    print(f"{wname}: {args.reps} calls of {g}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
