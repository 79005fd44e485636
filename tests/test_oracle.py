"""Pins for the fp64 CPU oracle: each test checks the oracle against something other
than itself -- brute force, a library routine, a closed form, an invariant, finite
differences or a hand-worked example -- chosen so that a dropped term, a wrong sign or
index, or a transposed operand fails at least one of them."""
import itertools
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import OShape
from conv2d_batchnorm_relu_amd.inputs import Geometry, draw

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def oshape(g: Geometry) -> OShape:
    return OShape(g.n, g.h, g.w, g.c, g.k, g.r, g.s, g.sh, g.sw, g.ph, g.pw)


def brute_conv(x, w, sh, sw, ph, pw):
    """Independent pure-Python loop nest (list indexing, no numpy arithmetic)."""
    N, H, W, C = x.shape
    K, R, S, _ = w.shape
    P = (H + 2 * ph - R) // sh + 1
    Q = (W + 2 * pw - S) // sw + 1
    xl, wl = x.tolist(), w.tolist()
    out = [[[[0.0] * K for _ in range(Q)] for _ in range(P)] for _ in range(N)]
    for n, p, q, k in itertools.product(range(N), range(P), range(Q), range(K)):
        acc = 0.0
        for r in range(R):
            for s in range(S):
                hh, ww = p * sh + r - ph, q * sw + s - pw
                if 0 <= hh < H and 0 <= ww < W:
                    for c in range(C):
                        acc += xl[n][hh][ww][c] * wl[k][r][s][c]
        out[n][p][q][k] = acc
    return np.array(out)


GEOMS = [
    Geometry(2, 8, 8, 4, 8, 3, 3, 1, 1),      # the tiny workload
    Geometry(1, 9, 11, 3, 4, 7, 7, 2, 3),     # stem-like 7x7 stride 2, Cin 3, odd sizes
    Geometry(2, 5, 6, 5, 3, 1, 1, 1, 0),      # 1x1
    Geometry(1, 7, 6, 2, 3, 3, 3, 2, 0),      # stride 2, no padding, ragged
    Geometry(1, 4, 4, 3, 2, 3, 3, 1, 2),      # padding wider than the filter reach
] + [
    # Anisotropic geometry: every axis pair differs (stride, padding, filter size, image
    # size), so an index that reads the other axis's stride or padding fails.
    Geometry(2, 9, 7, 3, 4, 3, 5, stride=2, pad=1, stride_w=1, pad_w=2),    # stride (2,1), pad (1,2), 3x5
    Geometry(1, 11, 6, 2, 3, 7, 1, stride=1, pad=3, stride_w=2, pad_w=0),   # 7x1, stride (1,2), pad (3,0)
    Geometry(1, 8, 10, 3, 2, 1, 3, stride=3, pad=0, stride_w=1, pad_w=1),   # 1x3, stride (3,1), pad (0,1)
]
ANISO = GEOMS[-3:]


@pytest.mark.parametrize("g", GEOMS, ids=str)
def test_conv_matches_brute_force(g):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((g.n, g.h, g.w, g.c))
    w = rng.standard_normal((g.k, g.r, g.s, g.c))
    z = oracle.conv2d(oshape(g), x, w)
    ref = brute_conv(x, w, g.sh, g.sw, g.ph, g.pw)
    assert z.shape == ref.shape == (g.n, g.p, g.q, g.k)
    np.testing.assert_allclose(z, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("g", GEOMS, ids=str)
def test_conv_matches_torch_conv2d(g):
    rng = np.random.default_rng(12)
    x = rng.standard_normal((g.n, g.h, g.w, g.c))
    w = rng.standard_normal((g.k, g.r, g.s, g.c))
    b = rng.standard_normal(g.k)
    z = oracle.conv2d(oshape(g), x, w, b)
    zt = F.conv2d(torch.from_numpy(x).permute(0, 3, 1, 2), torch.from_numpy(w).permute(0, 3, 1, 2),
                  torch.from_numpy(b), stride=(g.sh, g.sw), padding=(g.ph, g.pw)).permute(0, 2, 3, 1).numpy()
    np.testing.assert_allclose(z, zt, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("g", [GEOMS[0], GEOMS[3]] + ANISO[:1], ids=str)
def test_conv_bias_act_matches_brute_force(g):
    """Conv2D + bias (+ ReLU) without batch normalisation: the brute-force loop nest plus
    the bias, then max(., 0); a NULL bias adds nothing."""
    rng = np.random.default_rng(18)
    x = rng.standard_normal((g.n, g.h, g.w, g.c))
    w = rng.standard_normal((g.k, g.r, g.s, g.c))
    b = rng.standard_normal(g.k)
    ref = brute_conv(x, w, g.sh, g.sw, g.ph, g.pw)
    assert (ref + b < 0).any() and (ref + b > 0).any()
    sp = oshape(g)
    np.testing.assert_allclose(oracle.conv2d_bias_act(sp, x, w, b, relu=False), ref + b, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.conv2d_bias_act(sp, x, w, b, relu=True), np.maximum(ref + b, 0.0),
                               rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.conv2d_bias_act(sp, x, w, None, relu=True), np.maximum(ref, 0.0),
                               rtol=1e-13, atol=1e-13)


def test_conv_1x1_is_matmul():
    g = Geometry(3, 5, 7, 6, 4, 1, 1, 1, 0)
    rng = np.random.default_rng(13)
    x = rng.standard_normal((g.n, g.h, g.w, g.c))
    w = rng.standard_normal((g.k, 1, 1, g.c))
    z = oracle.conv2d(oshape(g), x, w)
    np.testing.assert_allclose(z.reshape(-1, g.k), x.reshape(-1, g.c) @ w.reshape(g.k, g.c).T,
                               rtol=1e-13, atol=1e-13)


def test_conv_centre_delta_is_identity():
    g = Geometry(2, 6, 5, 4, 4, 3, 3, 1, 1)
    rng = np.random.default_rng(14)
    x = rng.standard_normal((g.n, g.h, g.w, g.c))
    w = np.zeros((g.k, 3, 3, g.c))
    for k in range(g.k):
        w[k, 1, 1, k] = 1.0
    np.testing.assert_array_equal(oracle.conv2d(oshape(g), x, w), x)


@pytest.mark.parametrize("g", [Geometry(2, 9, 7, 5, 6, 3, 3, 2, 1)] + ANISO, ids=str)
def test_conv_at_matches_full(g):
    rng = np.random.default_rng(15)
    x = rng.standard_normal((g.n, g.h, g.w, g.c))
    w = rng.standard_normal((g.k, g.r, g.s, g.c))
    z = oracle.conv2d(oshape(g), x, w).ravel()
    idx = rng.choice(z.size, 50, replace=False)
    np.testing.assert_array_equal(oracle.conv2d_at(oshape(g), x, w, idx), z[idx])


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, rhs = line.split("=")
                vals[key.strip()] = np.array([float(v) for v in rhs.split()])
    return vals


def test_hand_worked_example():
    gv = _golden("hand_1x1.txt")
    sp = OShape(1, 1, 4, 1, 1, 1, 1, 1, 1, 0, 0)
    x = gv["x"].reshape(1, 1, 4, 1)
    w = gv["w"].reshape(1, 1, 1, 1)
    fw = oracle.forward_train(sp, x, w, [1.0], [0.0], [0.0], [1.0], 0.0, 0.1)
    tol = dict(rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fw["z"].ravel(), gv["z"], **tol)
    np.testing.assert_allclose(fw["mean"], gv["mean"], **tol)
    np.testing.assert_allclose(fw["var"], gv["var"], **tol)
    np.testing.assert_allclose(fw["invstd"], gv["invstd"], **tol)
    np.testing.assert_allclose(fw["y"].ravel(), gv["y"], **tol)
    np.testing.assert_array_equal(fw["mask"].ravel(), gv["mask"])
    np.testing.assert_allclose(fw["run_mean"], gv["run_mean"], **tol)
    np.testing.assert_allclose(fw["run_var"], gv["run_var"], **tol)
    bw = oracle.backward(sp, x, w, fw["z"], fw["mask"], gv["dy"].reshape(1, 1, 4, 1), [1.0],
                         fw["mean"], fw["invstd"])
    np.testing.assert_allclose(bw["dbeta"], gv["dbeta"], **tol)
    np.testing.assert_allclose(bw["dgamma"], gv["dgamma"], **tol)
    np.testing.assert_allclose(bw["dz"].ravel(), gv["dz"], **tol)
    np.testing.assert_allclose(bw["dw"].ravel(), gv["dw"], **tol)
    np.testing.assert_allclose(bw["dx"].ravel(), gv["dx"], **tol)
    y = oracle.forward_infer(sp, x, w, [0.5], [2.0], [-1.0], [1.0], [4.0], 0.0)
    np.testing.assert_allclose(y.ravel(), gv["infer_y"], **tol)
    wf, bf = oracle.fold(w, [0.5], [2.0], [-1.0], [1.0], [4.0], 0.0)
    np.testing.assert_allclose(wf.ravel(), gv["w_fold"], **tol)
    np.testing.assert_allclose(bf, gv["b_fold"], **tol)


def _tiny():
    g = Geometry(2, 8, 8, 4, 8, 3, 3, 1, 1)
    return g, {k: v.astype(np.float64) for k, v in draw(g, "train", 1, bf16=False).items()}


def test_train_stats_invariants():
    """With beta large enough that u > 0 everywhere, y = u; then per channel
    mean(u) = beta and var(u) = gamma^2 var/(var+eps) (BN output moments)."""
    g, d = _tiny()
    eps = 1e-5
    beta = d["beta"] + 50.0
    fw = oracle.forward_train(oshape(g), d["x"], d["w"], d["gamma"], beta, d["run_mean"], d["run_var"],
                              eps, 0.1)
    assert fw["mask"].all()
    u = fw["y"].reshape(-1, g.k)
    np.testing.assert_allclose(u.mean(0), beta, rtol=1e-13, atol=1e-12)
    np.testing.assert_allclose(u.var(0), d["gamma"] ** 2 * fw["var"] / (fw["var"] + eps), rtol=1e-12)
    # the batch statistics are those of z itself
    z = fw["z"].reshape(-1, g.k)
    np.testing.assert_allclose(fw["mean"], z.mean(0), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fw["var"], z.var(0), rtol=1e-12)


def test_train_matches_torch_batch_norm():
    g, d = _tiny()
    eps, mom = 1e-5, 0.1
    fw = oracle.forward_train(oshape(g), d["x"], d["w"], d["gamma"], d["beta"], d["run_mean"],
                              d["run_var"], eps, mom)
    zt = torch.from_numpy(fw["z"]).permute(0, 3, 1, 2)
    rm = torch.from_numpy(d["run_mean"].copy())
    rv = torch.from_numpy(d["run_var"].copy())
    u = F.batch_norm(zt, rm, rv, torch.from_numpy(d["gamma"]), torch.from_numpy(d["beta"]),
                     training=True, momentum=mom, eps=eps).permute(0, 2, 3, 1).numpy()
    np.testing.assert_allclose(fw["y"], np.maximum(u, 0), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(fw["mask"], (u > 0).astype(np.uint8))
    np.testing.assert_allclose(fw["run_mean"], rm.numpy(), rtol=1e-12, atol=1e-15)
    # torch's running variance is unbiased (M/(M-1)); the pages' finalize uses the biased
    # batch variance.  Undo torch's factor and compare.
    M = g.m
    torch_var_biased = (rv.numpy() - (1 - mom) * d["run_var"]) / mom * (M - 1) / M
    np.testing.assert_allclose(fw["var"], torch_var_biased, rtol=1e-10)
    np.testing.assert_allclose(fw["invstd"], 1 / np.sqrt(torch_var_biased + eps), rtol=1e-10)


def test_fold_identity():
    """relu(conv(x, w_fold) + b_fold) equals the inference definition."""
    g = Geometry(2, 7, 6, 5, 6, 3, 3, 1, 1)
    d = {k: v.astype(np.float64) for k, v in draw(g, "infer", 4, bf16=False).items()}
    eps = 1e-5
    y = oracle.forward_infer(oshape(g), d["x"], d["w"], d["bias"], d["gamma"], d["beta"],
                             d["run_mean"], d["run_var"], eps)
    wf, bf = oracle.fold(d["w"], d["bias"], d["gamma"], d["beta"], d["run_mean"], d["run_var"], eps)
    yf = np.maximum(oracle.conv2d(oshape(g), d["x"], wf, bf), 0)
    np.testing.assert_allclose(yf, y, rtol=1e-12, atol=1e-13)
    assert (y > 0).mean() > 0.2 and (y == 0).mean() > 0.2
    # and against torch's eval-mode batch_norm on the conv output
    zt = F.conv2d(torch.from_numpy(d["x"]).permute(0, 3, 1, 2), torch.from_numpy(d["w"]).permute(0, 3, 1, 2),
                  torch.from_numpy(d["bias"]), padding=1)
    ut = F.batch_norm(zt, torch.from_numpy(d["run_mean"]), torch.from_numpy(d["run_var"]),
                      torch.from_numpy(d["gamma"]), torch.from_numpy(d["beta"]), training=False, eps=eps)
    np.testing.assert_allclose(y, torch.relu(ut).permute(0, 2, 3, 1).numpy(), rtol=1e-12, atol=1e-12)


def _loss(g, x, w, gamma, beta, dy, eps):
    fw = oracle.forward_train(oshape(g), x, w, gamma, beta, np.zeros(g.k), np.ones(g.k), eps, 0.1)
    return float((fw["y"] * dy).sum()), fw


def test_backward_finite_differences():
    """Central differences of L = sum(dy * y) in x, w, gamma, beta (fp64, h = 1e-6)."""
    g, d = _tiny()
    eps, h = 1e-5, 1e-6
    x, w, gam, bet, dy = d["x"], d["w"], d["gamma"], d["beta"], d["dy"]
    _, fw = _loss(g, x, w, gam, bet, dy, eps)
    u_abs = np.abs(d["gamma"] * (fw["z"] - fw["mean"]) * fw["invstd"] + d["beta"])
    assert u_abs.min() > 1e-4, "seed puts a pre-activation on the ReLU kink"
    bw = oracle.backward(oshape(g), x, w, fw["z"], fw["mask"], dy, gam, fw["mean"], fw["invstd"])

    def fd(arr, grad, name):
        flat = arr.reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + h
            lp, _ = _loss(g, x, w, gam, bet, dy, eps)
            flat[i] = old - h
            lm, _ = _loss(g, x, w, gam, bet, dy, eps)
            flat[i] = old
            num = (lp - lm) / (2 * h)
            assert abs(num - grad.reshape(-1)[i]) <= 2e-6 * (1 + abs(num)), (name, i, num, grad.reshape(-1)[i])

    fd(x, bw["dx"], "dx")
    fd(w, bw["dw"], "dw")
    fd(gam, bw["dgamma"], "dgamma")
    fd(bet, bw["dbeta"], "dbeta")


def test_backward_matches_torch_autograd():
    g, d = _tiny()
    eps = 1e-5
    t = {k: torch.from_numpy(v.copy()) for k, v in d.items()}
    xt = t["x"].permute(0, 3, 1, 2).requires_grad_()
    wt = t["w"].permute(0, 3, 1, 2).requires_grad_()
    gt, bt = t["gamma"].requires_grad_(), t["beta"].requires_grad_()
    z = F.conv2d(xt, wt, padding=1)
    y = torch.relu(F.batch_norm(z, None, None, gt, bt, training=True, eps=eps))
    (y * t["dy"].permute(0, 3, 1, 2)).sum().backward()
    _, fw = _loss(g, d["x"], d["w"], d["gamma"], d["beta"], d["dy"], eps)
    bw = oracle.backward(oshape(g), d["x"], d["w"], fw["z"], fw["mask"], d["dy"], d["gamma"],
                         fw["mean"], fw["invstd"])
    tol = dict(rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(bw["dx"], xt.grad.permute(0, 2, 3, 1).numpy(), **tol)
    np.testing.assert_allclose(bw["dw"], wt.grad.permute(0, 2, 3, 1).numpy(), **tol)
    np.testing.assert_allclose(bw["dgamma"], gt.grad.numpy(), **tol)
    np.testing.assert_allclose(bw["dbeta"], bt.grad.numpy(), **tol)


def test_bn_backward_invariants():
    """sum_m dz = 0 and sum_m dz*xhat = gamma*invstd*dgamma*eps/(var+eps) per channel."""
    g, d = _tiny()
    eps = 1e-5
    _, fw = _loss(g, d["x"], d["w"], d["gamma"], d["beta"], d["dy"], eps)
    dz, dgam, dbet = oracle.bn_backward(d["dy"], fw["mask"], fw["z"], d["gamma"], fw["mean"], fw["invstd"])
    dz2 = dz.reshape(-1, g.k)
    xhat = ((fw["z"] - fw["mean"]) * fw["invstd"]).reshape(-1, g.k)
    scale = np.abs(dz2).sum(0)
    assert np.all(np.abs(dz2.sum(0)) <= 1e-13 * scale)
    expect = d["gamma"] * fw["invstd"] * dgam * eps / (fw["var"] + eps)
    np.testing.assert_allclose((dz2 * xhat).sum(0), expect, rtol=1e-6, atol=1e-13 * scale.max())
    g2 = (d["dy"] * fw["mask"]).reshape(-1, g.k)
    np.testing.assert_allclose(dbet, g2.sum(0), rtol=1e-13)
    assert (fw["mask"] == 0).any() and (fw["mask"] == 1).any()


@pytest.mark.parametrize("g", [Geometry(2, 8, 8, 4, 8, 3, 3, 1, 1), Geometry(2, 9, 11, 3, 5, 7, 7, 2, 3),
                               Geometry(1, 7, 6, 6, 4, 3, 3, 2, 0), Geometry(2, 5, 5, 3, 2, 1, 1, 1, 0)] + ANISO,
                         ids=str)
def test_dgrad_wgrad_adjointness(g):
    """<conv(x,w), dz> = <x, dgrad(dz,w)> = <w, wgrad(dz,x)> for an independent random dz."""
    rng = np.random.default_rng(16)
    x = rng.standard_normal((g.n, g.h, g.w, g.c))
    w = rng.standard_normal((g.k, g.r, g.s, g.c))
    dz = rng.standard_normal((g.n, g.p, g.q, g.k))
    sp = oshape(g)
    a = float((oracle.conv2d(sp, x, w) * dz).sum())
    b = float((x * oracle.conv2d_dgrad(sp, dz, w)).sum())
    c = float((w * oracle.conv2d_wgrad(sp, dz, x)).sum())
    assert abs(a - b) <= 1e-11 * (1 + abs(a))
    assert abs(a - c) <= 1e-11 * (1 + abs(a))


@pytest.mark.parametrize("g", [Geometry(2, 9, 11, 3, 5, 7, 7, 2, 3)] + ANISO, ids=str)
def test_dgrad_wgrad_match_torch(g):
    rng = np.random.default_rng(17)
    x = torch.from_numpy(rng.standard_normal((g.n, g.h, g.w, g.c)))
    w = torch.from_numpy(rng.standard_normal((g.k, g.r, g.s, g.c)))
    dz = torch.from_numpy(rng.standard_normal((g.n, g.p, g.q, g.k)))
    xt = x.permute(0, 3, 1, 2).clone().requires_grad_()
    wt = w.permute(0, 3, 1, 2).clone().requires_grad_()
    (F.conv2d(xt, wt, stride=(g.sh, g.sw), padding=(g.ph, g.pw)) * dz.permute(0, 3, 1, 2)).sum().backward()
    sp = oshape(g)
    np.testing.assert_allclose(oracle.conv2d_dgrad(sp, dz.numpy(), w.numpy()),
                               xt.grad.permute(0, 2, 3, 1).numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.conv2d_wgrad(sp, dz.numpy(), x.numpy()),
                               wt.grad.permute(0, 2, 3, 1).numpy(), rtol=1e-12, atol=1e-12)


def test_first_layer_backward_skips_dx():
    g, d = _tiny()
    _, fw = _loss(g, d["x"], d["w"], d["gamma"], d["beta"], d["dy"], 1e-5)
    full = oracle.backward(oshape(g), d["x"], d["w"], fw["z"], fw["mask"], d["dy"], d["gamma"],
                           fw["mean"], fw["invstd"])
    first = oracle.backward(oshape(g), d["x"], d["w"], fw["z"], fw["mask"], d["dy"], d["gamma"],
                            fw["mean"], fw["invstd"], want_dx=False)
    assert first["dx"] is None
    for k in ("dz", "dgamma", "dbeta", "dw"):
        np.testing.assert_array_equal(first[k], full[k])


def test_mask_is_strict_and_threshold_exact():
    """A 1x1 conv of evenly spaced values puts pre-activations on a fine grid through 0,
    one of them exactly 0: mask must be u > 0 strictly (CMP_GT), y = 0 at u = 0."""
    M = 20001
    x = np.arange(-(M // 2), M // 2 + 1, dtype=np.float64).reshape(1, 1, M, 1)  # mean exactly 0
    sp = OShape(1, 1, M, 1, 1, 1, 1, 1, 1, 0, 0)
    fw = oracle.forward_train(sp, x, np.ones((1, 1, 1, 1)), [1.0], [0.0], [0.0], [1.0], 0.0, 0.1)
    assert fw["mean"][0] == 0.0
    mask = fw["mask"].ravel()
    centre = M // 2
    assert x.ravel()[centre] == 0.0
    assert mask[centre] == 0 and fw["y"].ravel()[centre] == 0.0
    np.testing.assert_array_equal(mask[:centre], 0)
    np.testing.assert_array_equal(mask[centre + 1:], 1)
    np.testing.assert_array_equal(mask, (fw["y"].ravel() > 0).astype(np.uint8))
