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


def gpu_conv_bias(g: Geometry, x, w, bias, relu):
    """cbr_conv2d_bias_relu (relu) or cbr_conv2d_bias on host inputs; returns y."""
    import torch
    import conv2d_batchnorm_relu_amd as cbr
    y = empty_bf16((g.n, g.p, g.q, g.k))
    b = dev_f32(bias) if bias is not None else None
    fn = cbr.cbr_conv2d_bias_relu if relu else cbr.cbr_conv2d_bias
    fn(cshape(g), dev_bf16(x), dev_bf16(w), b, y)
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


def check_train(g: Geometry, d: dict, res: dict, ora: dict, eps=1e-5, momentum=0.1, y_from_stored_z=False):
    """Element-by-element comparison of a training forward with the oracle.

    With y_from_stored_z, y and the mask are compared with the oracle's normalisation
    (its statistics, gamma, beta) applied to the GPU's stored bf16 z rather than to the
    oracle's own z: for channels whose mean is many standard deviations from zero, the
    bf16 rounding of z alone moves u by up to |mean| * invstd * gamma * 2^-9."""
    M = g.m
    assert_close(res["z"], ora["z"], "z")
    zu = res["z"].astype(np.float64) if y_from_stored_z else ora["z"]
    u = d["gamma"].astype(np.float64) * (zu - ora["mean"]) * ora["invstd"] + d["beta"]
    assert_close(res["y"], np.maximum(u, 0.0) if y_from_stored_z else ora["y"], "y")
    if y_from_stored_z:
        ora = dict(ora, mask=(u > 0).astype(np.uint8))
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
    """The oracle's backward fed the GPU forward's own saved state (z, mask, stats).
    Also returns the masked gradient g and xhat it formed (for the dz rounding check)."""
    ob = oracle.backward(oshape(g), d["x"], d["w"], res["z"], res["mask"], dy, d["gamma"],
                         res["mean"], res["invstd"], want_dx=want_dx)
    mean = res["mean"].astype(np.float64)
    inv = res["invstd"].astype(np.float64)
    ob["g"] = np.where(res["mask"] != 0, dy.astype(np.float64), 0.0)
    ob["xhat"] = (res["z"].astype(np.float64) - mean) * inv
    ob["invstd_used"] = inv
    return ob


def check_backward(g: Geometry, d: dict, bw: dict, ob: dict, want_dx=True):
    """dz, dgamma, dbeta against the oracle; dw and dx against the oracle's weight and
    data gradients of the call's own bf16 dz (the library's contract: both read the
    stored dz) to the bf16 tolerance, and end to end against the exact oracle.

    dz is also held to its rounding: the GPU computes it in fp32 and rounds it to bf16
    once, so |dz - dz_oracle| <= 2^-8 |dz_oracle| plus 1e-5 of the magnitude of the terms
    it is formed from (gamma * invstd * (|g| + |dbeta|/M + |xhat dgamma|/M)).

    End to end, the rounding of dz to bf16 moves dw = sum_m dz_m x_m by sum_m e_m dz_m x_m
    with independent relative errors |e_m| <= 2^-9 (round to nearest: uniform, standard
    deviation 2^-9/sqrt(3)).  dw and dx are held to the bf16 tolerance plus six standard
    deviations of that sum, 6 * 2^-9/sqrt(3) * sqrt(sum_m (dz_m x_m)^2), which grows like
    sqrt(M).  The largest end-to-end error and the share of elements inside the plain
    tolerance are returned."""
    assert bw["dz"] is not None, "run the backward with a dz output to check it"
    assert_close(bw["dz"], ob["dz"], "dz")
    gam = d["gamma"].astype(np.float64)
    inv = ob["invstd_used"] if "invstd_used" in ob else None
    assert_close(bw["dbeta"], ob["dbeta"], "dbeta")
    assert_close(bw["dgamma"], ob["dgamma"], "dgamma")
    if inv is not None:
        M = g.m
        terms = gam * inv * (np.abs(ob["g"]) + np.abs(ob["dbeta"]) / M + np.abs(ob["xhat"] * ob["dgamma"]) / M)
        dz_err = np.abs(bw["dz"] - ob["dz"])
        bad = dz_err > 2.0 ** -8 * np.abs(ob["dz"]) + 1e-5 * terms
        assert not bad.any(), f"dz beyond its bf16 rounding: {int(bad.sum())} of {bad.size}"
    sp = oshape(g)
    dw_on_dz = oracle.conv2d_wgrad(sp, bw["dz"], d["x"])
    assert_close(bw["dw"], dw_on_dz, "dw (oracle on the stored dz)")
    sd = 2.0 ** -9 / np.sqrt(3.0)
    dz2 = bw["dz"].astype(np.float64) ** 2
    bound_w = 6.0 * sd * np.sqrt(oracle.conv2d_wgrad(sp, dz2, d["x"].astype(np.float64) ** 2))
    err = np.abs(bw["dw"] - ob["dw"])
    tol = BF16_ATOL + BF16_RTOL * np.abs(ob["dw"])
    assert (err <= tol + bound_w).all(), \
        f"dw end to end: max excess {float((err - bound_w - tol).max())}"
    out = dict(dw_max_err=float(err.max()), dw_within_tol=float((err <= tol).mean()))
    if want_dx:
        dx_on_dz = oracle.conv2d_dgrad(sp, bw["dz"], d["w"])
        assert_close(bw["dx"], dx_on_dz, "dx (oracle on the stored dz)")
        bound_x = 6.0 * sd * np.sqrt(oracle.conv2d_dgrad(sp, dz2, d["w"].astype(np.float64) ** 2))
        errx = np.abs(bw["dx"] - ob["dx"])
        tolx = BF16_ATOL + BF16_RTOL * np.abs(ob["dx"])
        assert (errx <= tolx + bound_x).all(), \
            f"dx end to end: max excess {float((errx - bound_x - tolx).max())}"
        out.update(dx_max_err=float(errx.max()), dx_within_tol=float((errx <= tolx).mean()))
    log(f"end to end: {out}")
    return out
