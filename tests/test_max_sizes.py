"""The training forward at the largest batch the ABI accepts (every tensor just under 2^30
elements), one layer per forward kernel family: the persistent 3x3 / 64-channel conv, the
first-layer conv and the large-tile conv.  The batch repeats PERIOD seeded images (image n
is base image n % PERIOD), so the oracle computes only the base images:
  - the base images' z, y and mask against the oracle element by element;
  - every other image's z, y and mask equal to its base image's, bit for bit (the kernels
    are deterministic and each output pixel's arithmetic does not depend on where it sits
    in the batch), which checks every image the batch holds;
  - the batch statistics against their definition (mean = sum z / M, var = sum (z - mean)^2
    / M) over the oracle's base images, each counted as often as it repeats, to the same
    bounds as the other tests.
This exercises the index arithmetic (step ranges crossing hundreds of images, byte offsets
near 2^31, the statistics rows of every workgroup) at the sizes where it could overflow.
A period of 7 images does not divide the per-image byte or step strides of these layers,
so an index that lands on the wrong image reads different data."""
import numpy as np
import pytest

from conv2d_batchnorm_relu_amd.inputs import Geometry, draw
import cbr_harness as H
import oracle

pytestmark = pytest.mark.gpu

MAX_ELEMS = 1 << 30   # the ABI rejects any tensor with this many elements or more
PERIOD = 7

MAX_GEOMS = [
    Geometry(5349, 56, 56, 64, 64, 3, 3, 1, 1),     # persistent 3x3 / 64-channel conv
    Geometry(1337, 224, 224, 3, 64, 7, 7, 2, 3),    # first-layer conv
    Geometry(21399, 14, 14, 256, 256, 3, 3, 1, 1),  # large-tile conv (224 x 256 chunks)
]


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import conv2d_batchnorm_relu_amd as cbr
    cbr._load()


@pytest.mark.parametrize("g", MAX_GEOMS, ids=str)
def test_train_forward_max_batch(g):
    import torch
    import conv2d_batchnorm_relu_amd as cbr
    assert max(g.n * g.h * g.w * g.c, g.m * g.k) < MAX_ELEMS
    assert max((g.n + 1) * g.h * g.w * g.c, (g.n + 1) * g.p * g.q * g.k) >= MAX_ELEMS   # the largest N
    eps, momentum = 1e-5, 0.1
    gb = Geometry(PERIOD, g.h, g.w, g.c, g.k, g.r, g.s, g.stride, g.pad, g.stride_w, g.pad_w)
    d = draw(gb, "train", 61)
    H.log(f"max batch {g}, period {PERIOD}")

    xb = H.dev_bf16(d["x"])
    reps = -(-g.n // PERIOD)
    x = xb.repeat(reps, 1, 1, 1)[:g.n].contiguous()
    w = H.dev_bf16(d["w"])
    gamma, beta = H.dev_f32(d["gamma"]), H.dev_f32(d["beta"])
    rm_in, rv_in = H.dev_f32(d["run_mean"]), H.dev_f32(d["run_var"])
    sp = H.cshape(g)
    z = H.empty_bf16((g.n, g.p, g.q, g.k))
    y = H.empty_bf16((g.n, g.p, g.q, g.k))
    mask = torch.full((cbr.cbr_mask_words(sp),), -1, dtype=torch.int32, device="cuda")
    smean, sinv, rm_out, rv_out = (H.empty_f32(g.k) for _ in range(4))
    ws = H.workspace(cbr.cbr_workspace_bytes(sp, cbr.CBR_OP_TRAIN))
    cbr.cbr_forward_train(sp, x, w, gamma, beta, rm_in, rv_in, eps, momentum, z, y, mask, smean, sinv,
                          rm_out, rv_out, ws)
    torch.cuda.synchronize()
    del x
    H.log("oracle on the base images")

    # oracle: conv of the base images; statistics of the whole batch by definition, base
    # image b counted once per image n with n % PERIOD == b
    zb = oracle.conv2d(H.oshape(gb), d["x"], d["w"])                   # [PERIOD, P, Q, K] fp64
    times = np.array([len(range(b, g.n, PERIOD)) for b in range(PERIOD)], np.float64)
    M = g.m
    per_img = zb.reshape(PERIOD, -1, g.k)
    mean = (times[:, None] * per_img.sum(axis=1)).sum(axis=0) / M
    var = (times[:, None] * ((per_img - mean) ** 2).sum(axis=1)).sum(axis=0) / M
    invstd = 1.0 / np.sqrt(var + eps)
    run_mean = (1 - momentum) * d["run_mean"] + momentum * mean
    run_var = (1 - momentum) * d["run_var"] + momentum * var

    # statistics
    mean_bound = H.STAT_RTOL * np.maximum(np.abs(mean), np.sqrt(var + eps) / np.sqrt(M))
    assert (np.abs(smean.cpu().numpy() - mean) <= mean_bound).all(), ("mean", smean.cpu().numpy(), mean)
    H.assert_close(sinv.cpu().numpy(), invstd, "invstd", rtol=H.STAT_RTOL, atol=0.0)
    rm_bound = momentum * mean_bound + H.STAT_RTOL * np.abs((1 - momentum) * d["run_mean"])
    assert (np.abs(rm_out.cpu().numpy() - run_mean) <= rm_bound + 1e-12).all(), "running mean"
    H.assert_close(rv_out.cpu().numpy(), run_var, "running var", rtol=H.STAT_RTOL, atol=0.0)

    # the base images (the batch's first PERIOD) against the oracle
    H.assert_close(H.host_bf16(z[:PERIOD]), zb, "z (base images)")
    ub = d["gamma"].astype(np.float64) * (zb - mean) * invstd + d["beta"]
    H.assert_close(H.host_bf16(y[:PERIOD]), np.maximum(ub, 0.0), "y (base images)")
    words_pp = g.k // 32                                               # mask words per pixel (K % 32 == 0)
    mwords = mask.view(g.n, g.p * g.q * words_pp)
    bits = H.unpack_mask(mwords[:PERIOD].reshape(-1), PERIOD * g.p * g.q * g.k).reshape(ub.shape)
    flips = bits != (ub > 0)
    assert not (flips & (np.abs(ub) > H.MASK_BAND)).any(), "mask (base images)"

    # every other image bit for bit equal to its base image
    zl, yl = z.view(g.n, -1), y.view(g.n, -1)
    bad = {"z": 0, "y": 0, "mask": 0}
    chunk = PERIOD * max(1, (1 << 26) // (PERIOD * g.p * g.q * g.k))
    for n0 in range(PERIOD, g.n, chunk):
        n1 = min(g.n, n0 + chunk)
        base = torch.arange(n0, n1, device="cuda") % PERIOD
        for name, t in (("z", zl), ("y", yl), ("mask", mwords)):
            bad[name] += int((t[n0:n1] != t[base]).any(dim=1).sum())
    assert bad == {"z": 0, "y": 0, "mask": 0}, f"images that differ from their base image: {bad}"
    H.log("ok")


def test_backward_max_batch():
    """The backward of the 14x14x256 layer at the largest batch (N = 21 399: dz, dx and x
    just under 2^30 elements), on a repeating batch of PERIOD images (x and dy).  Per base
    image the oracle gives dgamma and dbeta (bn_backward on that image alone); the batch's
    are their sums weighted by how often each base image repeats.  dz of a base image is
    then the definition dz = gamma * invstd * (g - dbeta/M - xhat * dgamma/M) with those
    sums; dw is the weighted sum of the oracle's weight gradients of the base images on the
    GPU's stored dz, dx of a base image the oracle's data gradient of its stored dz (the
    contract: both gradients read the stored bf16 dz).  Every other image's dz and dx must
    equal its base image's bit for bit."""
    import torch
    import conv2d_batchnorm_relu_amd as cbr
    g = Geometry(21399, 14, 14, 256, 256, 3, 3, 1, 1)
    assert max(g.n * g.h * g.w * g.c, g.m * g.k) < MAX_ELEMS
    eps, momentum = 1e-5, 0.1
    gb = Geometry(PERIOD, g.h, g.w, g.c, g.k, g.r, g.s, g.stride, g.pad)
    d = draw(gb, "bwd", 62)
    H.log(f"max batch backward {g}, period {PERIOD}")
    reps = -(-g.n // PERIOD)
    x = H.dev_bf16(d["x"]).repeat(reps, 1, 1, 1)[:g.n].contiguous()
    dy = H.dev_bf16(d["dy"]).repeat(reps, 1, 1, 1)[:g.n].contiguous()
    w = H.dev_bf16(d["w"])
    gamma, beta = H.dev_f32(d["gamma"]), H.dev_f32(d["beta"])
    rm, rv = H.dev_f32(d["run_mean"]), H.dev_f32(d["run_var"])
    sp = H.cshape(g)
    z = H.empty_bf16((g.n, g.p, g.q, g.k))
    y = H.empty_bf16((g.n, g.p, g.q, g.k))
    mask = torch.zeros((cbr.cbr_mask_words(sp),), dtype=torch.int32, device="cuda")
    smean, sinv, rm_out, rv_out = (H.empty_f32(g.k) for _ in range(4))
    ws = H.workspace(max(cbr.cbr_workspace_bytes(sp, cbr.CBR_OP_TRAIN), cbr.cbr_workspace_bytes(sp, cbr.CBR_OP_BWD)))
    cbr.cbr_forward_train(sp, x, w, gamma, beta, rm, rv, eps, momentum, z, y, mask, smean, sinv, rm_out, rv_out, ws)
    del y
    dz = H.empty_bf16((g.n, g.p, g.q, g.k))
    dx = H.empty_bf16((g.n, g.h, g.w, g.c))
    dgam, dbet = H.empty_f32(g.k), H.empty_f32(g.k)
    dw = H.empty_f32((g.k, g.r, g.s, g.c))
    cbr.cbr_backward(sp, x, w, z, mask, dy, gamma, smean, sinv, dz, dgam, dbet, dw, dx, ws)
    torch.cuda.synchronize()
    H.log("oracle on the base images")

    # the GPU forward's state of the base images (the batch's first PERIOD)
    zb = H.host_bf16(z[:PERIOD])
    words_pp = g.k // 32
    mwords = mask.view(g.n, g.p * g.q * words_pp)
    mb = H.unpack_mask(mwords[:PERIOD].reshape(-1), PERIOD * g.p * g.q * g.k).reshape(zb.shape)
    mean, inv = smean.cpu().numpy().astype(np.float64), sinv.cpu().numpy().astype(np.float64)
    times = np.array([len(range(b, g.n, PERIOD)) for b in range(PERIOD)], np.float64)
    M = g.m
    dgs, dbs = [], []
    for b in range(PERIOD):
        _, dg_b, db_b = oracle.bn_backward(d["dy"][b], mb[b], zb[b], d["gamma"], mean, inv)
        dgs.append(dg_b)
        dbs.append(db_b)
    dgamma = (times[:, None] * np.array(dgs)).sum(axis=0)
    dbeta = (times[:, None] * np.array(dbs)).sum(axis=0)
    H.assert_close(dgam.cpu().numpy(), dgamma, "dgamma")
    H.assert_close(dbet.cpu().numpy(), dbeta, "dbeta")
    gmask = np.where(mb != 0, d["dy"].astype(np.float64), 0.0)
    xhat = (zb.astype(np.float64) - mean) * inv
    dz_def = d["gamma"].astype(np.float64) * inv * (gmask - dbeta / M - xhat * dgamma / M)
    dzb = H.host_bf16(dz[:PERIOD])
    H.assert_close(dzb, dz_def, "dz (base images)")

    spb = H.oshape(gb)
    dw_ref = np.zeros((g.k, g.r, g.s, g.c))
    for b in range(PERIOD):
        spi = H.oshape(Geometry(1, g.h, g.w, g.c, g.k, g.r, g.s, g.stride, g.pad))
        dw_ref += times[b] * oracle.conv2d_wgrad(spi, dzb[b:b + 1], d["x"][b:b + 1])
    H.assert_close(dw.cpu().numpy(), dw_ref, "dw (weighted oracle on the stored dz)")
    H.assert_close(H.host_bf16(dx[:PERIOD]), oracle.conv2d_dgrad(spb, dzb, d["w"]), "dx (base images)")

    bad = {"dz": 0, "dx": 0}
    for name, t in (("dz", dz.view(g.n, -1)), ("dx", dx.view(g.n, -1))):
        chunk = PERIOD * max(1, (1 << 26) // (PERIOD * t.shape[1]))
        for n0 in range(PERIOD, g.n, chunk):
            n1 = min(g.n, n0 + chunk)
            base = torch.arange(n0, n1, device="cuda") % PERIOD
            bad[name] += int((t[n0:n1] != t[base]).any(dim=1).sum())
    assert bad == {"dz": 0, "dx": 0}, f"images that differ from their base image: {bad}"
    H.log("ok")
