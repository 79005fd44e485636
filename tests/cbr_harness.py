"""Test-side harness: runs the HIP library through its Python binding on seeded inputs,
runs the fp64 oracle on the same inputs, and compares them to the stated tolerances.

Tolerances (written here, used by every parity test):
  bf16 tensors and all gradients (z, y, dz, dx, dw, dgamma, dbeta):
      |gpu - oracle| <= 2e-2 + 2e-2 * |oracle|
  fp32 statistics: invstd, running variance: |gpu - oracle| <= 1e-4 * |oracle|;
      batch mean:    |gpu - oracle| <= 1e-4 * max(|oracle|, sqrt(var + eps) / sqrt(M))
      running mean:  the mean bound times momentum (plus the relative bound on the
                     (1 - momentum) * old part)
  ReLU mask: a bit may differ from the oracle's only where the oracle's pre-activation
      satisfies |u| <= 2e-2 (the GPU normalises the bf16-rounded conv output).
"""
from __future__ import annotations

import sys
import time

import numpy as np

import oracle
from conv2d_batchnorm_relu_amd.inputs import Geometry, bf16_bits, bf16_to_f32

BF16_RTOL = 2e-2
BF16_ATOL = 2e-2
STAT_RTOL = 1e-4
MASK_BAND = 2e-2


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def oshape(g: Geometry):
    return oracle.OShape(g.n, g.h, g.w, g.c, g.k, g.r, g.s, g.sh, g.sw, g.ph, g.pw)


def cshape(g: Geometry):
    import conv2d_batchnorm_relu_amd as cbr
    return cbr.make_shape(g.n, g.h, g.w, g.c, g.k, g.r, g.s, g.sh, g.ph, stride_w=g.sw, pad_w=g.pw)


def dev_bf16(a, device="cuda"):
    import torch
    return torch.from_numpy(bf16_bits(a).view(np.int16)).to(device)


def dev_f32(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host_bf16(t):
    return bf16_to_f32(t.cpu().numpy().view(np.uint16))


def unpack_mask(words, count):
    w = np.ascontiguousarray(words.cpu().numpy()).view(np.uint8)
    return np.unpackbits(w, bitorder="little")[:count]


def empty_bf16(shape, device="cuda"):
    import torch
    return torch.empty(shape, dtype=torch.int16, device=device)


def empty_f32(shape, device="cuda"):
    import torch
    return torch.empty(shape, dtype=torch.float32, device=device)


def workspace(nbytes, device="cuda"):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------------
# GPU calls
# ----------------------------------------------------------------------------------

def gpu_train(g: Geometry, d: dict, eps=1e-5, momentum=0.1, inplace_running=False, dev=None):
    """Runs cbr_forward_train; returns host results and the device tensors."""
    import torch
    import conv2d_batchnorm_relu_amd as cbr
    sp = cshape(g)
    x = dev["x"] if dev and "x" in dev else dev_bf16(d["x"])
    w = dev["w"] if dev and "w" in dev else dev_bf16(d["w"])
    gamma, beta = dev_f32(d["gamma"]), dev_f32(d["beta"])
    rm_in, rv_in = dev_f32(d["run_mean"]), dev_f32(d["run_var"])
    z = empty_bf16((g.n, g.p, g.q, g.k))
    y = empty_bf16((g.n, g.p, g.q, g.k))
    mask = torch.full((cbr.cbr_mask_words(sp),), -1, dtype=torch.int32, device="cuda")
    smean, sinv = empty_f32(g.k), empty_f32(g.k)
    rm_out, rv_out = (rm_in, rv_in) if inplace_running else (empty_f32(g.k), empty_f32(g.k))
    ws = workspace(cbr.cbr_workspace_bytes(sp, cbr.CBR_OP_TRAIN))
    cbr.cbr_forward_train(sp, x, w, gamma, beta, rm_in, rv_in, eps, momentum, z, y, mask, smean, sinv,
                          rm_out, rv_out, ws)
    torch.cuda.synchronize()
    res = dict(z=host_bf16(z), y=host_bf16(y), mask_words=mask.cpu().numpy().view(np.uint32),
               mask=unpack_mask(mask, g.m * g.k).reshape(g.n, g.p, g.q, g.k),
               mean=smean.cpu().numpy(), invstd=sinv.cpu().numpy(),
               run_mean=rm_out.cpu().numpy(), run_var=rv_out.cpu().numpy())
    devt = dict(x=x, w=w, z=z, y=y, mask=mask, smean=smean, sinv=sinv, gamma=gamma)
    return res, devt


def gpu_infer(g: Geometry, d: dict, eps=1e-5):
    import torch
    import conv2d_batchnorm_relu_amd as cbr
    sp = cshape(g)
    y = empty_bf16((g.n, g.p, g.q, g.k))
    bias = dev_f32(d["bias"]) if d.get("bias") is not None else None
    ws = workspace(cbr.cbr_workspace_bytes(sp, cbr.CBR_OP_INFER))
    cbr.cbr_forward_infer(sp, dev_bf16(d["x"]), dev_bf16(d["w"]), bias, dev_f32(d["gamma"]),
                          dev_f32(d["beta"]), dev_f32(d["run_mean"]), dev_f32(d["run_var"]), eps, y, ws)
    torch.cuda.synchronize()
    return host_bf16(y)


def gpu_backward(g: Geometry, devt: dict, dy_host, want_dx=True, dz_out=True, dx_alias_x=False):
    import torch
    import conv2d_batchnorm_relu_amd as cbr
    sp = cshape(g)
    dy = dev_bf16(dy_host)
    dz = empty_bf16((g.n, g.p, g.q, g.k)) if dz_out else None
    dgam, dbet = empty_f32(g.k), empty_f32(g.k)
    dw = empty_f32((g.k, g.r, g.s, g.c))
    if dx_alias_x:
        dx = devt["x"]
    else:
        dx = empty_bf16((g.n, g.h, g.w, g.c)) if want_dx else None
    ws = workspace(cbr.cbr_workspace_bytes(sp, cbr.CBR_OP_BWD))
    cbr.cbr_backward(sp, devt["x"], devt["w"], devt["z"], devt["mask"], dy, devt["gamma"], devt["smean"],
                     devt["sinv"], dz, dgam, dbet, dw, dx, ws)
    torch.cuda.synchronize()
    return dict(dz=host_bf16(dz) if dz is not None else None, dgamma=dgam.cpu().numpy(),
                dbeta=dbet.cpu().numpy(), dw=dw.cpu().numpy(),
                dx=host_bf16(dx) if dx is not None else None)


# ----------------------------------------------------------------------------------
# comparisons
# ----------------------------------------------------------------------------------

def assert_close(gpu, ref, what, rtol=BF16_RTOL, atol=BF16_ATOL):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        i = np.flatnonzero(bad.ravel())[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at {i}: "
                             f"gpu={gpu.ravel()[i]} oracle={ref.ravel()[i]}")
    assert np.isfinite(gpu).all(), what
    return float(err.max()) if err.size else 0.0


def check_train(g: Geometry, d: dict, res: dict, ora: dict, eps=1e-5, momentum=0.1):
    """Element-by-element comparison of a training forward with the oracle."""
    M = g.m
    assert_close(res["z"], ora["z"], "z")
    assert_close(res["y"], ora["y"], "y")
    u = d["gamma"].astype(np.float64) * (ora["z"] - ora["mean"]) * ora["invstd"] + d["beta"]
    flips = res["mask"] != ora["mask"]
    assert not (flips & (np.abs(u) > MASK_BAND)).any(), \
        f"mask differs where |u| > {MASK_BAND}: {int((flips & (np.abs(u) > MASK_BAND)).sum())}"
    # packed-mask tail bits past M*K are zero
    nbits = M * g.k
    words = res["mask_words"]
    if nbits % 32:
        assert (int(words[-1]) >> (nbits % 32)) == 0, "mask tail bits not cleared"
    # mask consistent with y
    assert ((res["y"] > 0) == (res["mask"] == 1)).all(), "mask disagrees with y > 0"
    mean_bound = STAT_RTOL * np.maximum(np.abs(ora["mean"]), np.sqrt(ora["var"] + eps) / np.sqrt(M))
    assert (np.abs(res["mean"] - ora["mean"]) <= mean_bound).all(), ("mean", res["mean"], ora["mean"])
    assert_close(res["invstd"], ora["invstd"], "invstd", rtol=STAT_RTOL, atol=0.0)
    rm_bound = momentum * mean_bound + STAT_RTOL * np.abs((1 - momentum) * d["run_mean"])
    assert (np.abs(res["run_mean"] - ora["run_mean"]) <= rm_bound + 1e-12).all(), "running mean"
    assert_close(res["run_var"], ora["run_var"], "running var", rtol=STAT_RTOL, atol=0.0)
    return int(flips.sum())


def oracle_train(g: Geometry, d: dict, eps=1e-5, momentum=0.1):
    return oracle.forward_train(oshape(g), d["x"], d["w"], d["gamma"], d["beta"], d["run_mean"],
                                d["run_var"], eps, momentum)


def oracle_backward_on_gpu_state(g: Geometry, d: dict, res: dict, dy, want_dx=True):
    """The oracle's backward fed the GPU forward's own saved state (z, mask, stats)."""
    return oracle.backward(oshape(g), d["x"], d["w"], res["z"], res["mask"], dy, d["gamma"],
                           res["mean"], res["invstd"], want_dx=want_dx)


def check_backward(g: Geometry, d: dict, bw: dict, ob: dict, want_dx=True):
    """dz, dgamma, dbeta against the oracle; dw and dx against the oracle's weight and
    data gradients of the call's own bf16 dz (the library's contract: both read the
    stored dz), and end to end against the exact oracle within the bound that rounding
    dz to bf16 (relative error <= 2^-8) can move a sum of products:
    |delta dw| <= 2^-8 * sum_m |dz_m x_m|, |delta dx| <= 2^-8 * sum |dz w|."""
    assert bw["dz"] is not None, "run the backward with a dz output to check it"
    assert_close(bw["dz"], ob["dz"], "dz")
    assert_close(bw["dbeta"], ob["dbeta"], "dbeta")
    assert_close(bw["dgamma"], ob["dgamma"], "dgamma")
    sp = oshape(g)
    dw_on_dz = oracle.conv2d_wgrad(sp, bw["dz"], d["x"])
    assert_close(bw["dw"], dw_on_dz, "dw (oracle on the stored dz)")
    bound_w = 2.0 ** -8 * oracle.conv2d_wgrad(sp, np.abs(bw["dz"]), np.abs(d["x"]))
    err = np.abs(bw["dw"] - ob["dw"])
    assert (err <= BF16_ATOL + BF16_RTOL * np.abs(ob["dw"]) + bound_w).all(), \
        f"dw end to end: max excess {float((err - bound_w - BF16_ATOL - BF16_RTOL * np.abs(ob['dw'])).max())}"
    if want_dx:
        dx_on_dz = oracle.conv2d_dgrad(sp, bw["dz"], d["w"])
        assert_close(bw["dx"], dx_on_dz, "dx (oracle on the stored dz)")
        bound_x = 2.0 ** -8 * oracle.conv2d_dgrad(sp, np.abs(bw["dz"]), np.abs(d["w"]))
        errx = np.abs(bw["dx"] - ob["dx"])
        assert (errx <= BF16_ATOL + BF16_RTOL * np.abs(ob["dx"]) + bound_x).all(), "dx end to end"
