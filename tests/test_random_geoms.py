"""GPU parity on seeded random small geometries: channels (including odd counts, which take
the generic conv's element gather), filter sizes, strides and paddings drawn per axis, so
the plan choices and the kernels' edge handling meet shapes no fixed test names.  Each
geometry runs the training forward, the folded-BN inference and the backward (the data
gradient where the stride is 1) against the oracle, to the same bounds as the fixed tests."""
import numpy as np
import pytest

from conv2d_batchnorm_relu_amd.inputs import Geometry, draw
import cbr_harness as H

pytestmark = pytest.mark.gpu

CHANNELS_IN = [1, 3, 4, 5, 8, 12, 16, 24, 32, 40, 64, 128, 256]
CHANNELS_OUT = [8, 16, 24, 32, 40, 64, 72, 128, 136, 256]


def random_geometries(count, seed=2024, max_macs=40_000_000):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        r, s = (int(v) for v in rng.integers(1, 8, 2))
        sh, sw = (int(v) for v in rng.integers(1, 4, 2))
        ph, pw = int(rng.integers(0, r)), int(rng.integers(0, s))
        h = int(rng.integers(max(1, r - 2 * ph), 22))
        w = int(rng.integers(max(1, s - 2 * pw), 22))
        n = int(rng.integers(1, 4))
        c = int(rng.choice(CHANNELS_IN))
        k = int(rng.choice(CHANNELS_OUT))
        g = Geometry(n, h, w, c, k, r, s, sh, ph, stride_w=sw, pad_w=pw)
        if h + 2 * ph < r or w + 2 * pw < s or g.m < 2:
            continue
        if g.m * k * r * s * c > max_macs:
            continue
        out.append(g)
    return out


GEOMS = random_geometries(32)


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import conv2d_batchnorm_relu_amd as cbr
    cbr._load()


@pytest.mark.parametrize("g", GEOMS, ids=str)
def test_random_geometry(g):
    import ctypes
    import conv2d_batchnorm_relu_amd as cbr
    lib = cbr._load()
    lib.cbr_plan_name.restype = ctypes.c_char_p
    sp = H.cshape(g)
    plans = [lib.cbr_plan_name(lib.cbr_plan_of(ctypes.byref(sp), st)).decode() for st in range(5)]
    H.log(f"random {g} plans {plans}")
    d = draw(g, "bwd", 91)
    res, devt = H.gpu_train(g, d)
    ora = H.oracle_train(g, d)
    H.check_train(g, d, res, ora)

    di = draw(g, "infer", 92)
    y = H.gpu_infer(g, di)
    ref = H.oracle.forward_infer(H.oshape(g), di["x"], di["w"], di["bias"], di["gamma"], di["beta"],
                                 di["run_mean"], di["run_var"], 1e-5)
    H.assert_close(y, ref, "infer y")

    want_dx = g.sh == 1 and g.sw == 1
    bw = H.gpu_backward(g, devt, d["dy"], want_dx=want_dx)
    ob = H.oracle_backward_on_gpu_state(g, d, res, d["dy"], want_dx=want_dx)
    H.check_backward(g, d, bw, ob, want_dx)
