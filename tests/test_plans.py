"""Every kernel plan the tuner may force, on every stage it is eligible for, against the
oracle: the training forward's conv, the inference conv (conv + bias + ReLU), the data
gradient and the weight gradient.  Shapes are chosen so that each plan runs somewhere,
including the forms the default rule never picks (a 128-channel tile on a 64-channel
layer, 224 x 256 chunks with several pixel chunks and with two channel chunks)."""
import ctypes

import numpy as np
import pytest

from conv2d_batchnorm_relu_amd.inputs import Geometry, draw
import cbr_harness as H

pytestmark = pytest.mark.gpu

PLAN_GEOMS = [
    Geometry(2, 12, 16, 64, 64, 3, 3, 1, 1),       # persistent 3x3; generic 128x128 on K = 64
    Geometry(2, 32, 32, 3, 64, 7, 7, 2, 3),        # first layer
    Geometry(2, 9, 12, 64, 256, 3, 3, 1, 1),       # large tile both forms; generic both tiles
    Geometry(2, 10, 12, 128, 256, 3, 1, 1, 1, pad_w=0),   # transposed-read weight gradient; dgrad large tile
    Geometry(4, 20, 20, 64, 512, 1, 1, 1, 0),      # 224 x 256 chunks, two channel chunks
    Geometry(32, 56, 56, 64, 256, 1, 1, 1, 0),     # 224 x 256 chunks, two pixel chunks per workgroup
]


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def lib():
    import conv2d_batchnorm_relu_amd as cbr
    L = cbr._load()
    L.cbr_plan_name.restype = ctypes.c_char_p
    return L


def all_plans():
    """Every plan id the library names (ids run from 1 without gaps)."""
    out = []
    for p in range(1, 64):
        if lib().cbr_plan_name(p).decode() == "unknown":
            break
        out.append(p)
    return out


def eligible(g, stage):
    sp = H.cshape(g)
    return [p for p in all_plans() if lib().cbr_plan_eligible(ctypes.byref(sp), stage, p) == 1]


class forced:
    def __init__(self, stage, plan):
        self.stage, self.plan = stage, plan

    def __enter__(self):
        assert lib().cbr_set_plan_override(self.stage, self.plan) == 0

    def __exit__(self, *a):
        lib().cbr_set_plan_override(self.stage, 0)


def cases(stage):
    out = []
    for g in PLAN_GEOMS:
        if stage == 2 and (g.sh != 1 or g.sw != 1):
            continue
        for p in eligible_static(g, stage):
            out.append((g, p))
    return out


def eligible_static(g, stage):
    try:
        return eligible(g, stage)
    except Exception:   # library not built: collected anyway, skipped by the fixture
        return []


@pytest.mark.parametrize("g,plan", cases(0), ids=str)
def test_train_conv_plan(g, plan):
    H.log(f"train conv plan {lib().cbr_plan_name(plan).decode()} {g}")
    d = draw(g, "train", 41)
    with forced(0, plan):
        assert lib().cbr_plan_of(ctypes.byref(H.cshape(g)), 0) == plan
        res, _ = H.gpu_train(g, d)
    H.check_train(g, d, res, H.oracle_train(g, d))


@pytest.mark.parametrize("g,plan", cases(1), ids=str)
def test_infer_conv_plan(g, plan):
    H.log(f"infer conv plan {lib().cbr_plan_name(plan).decode()} {g}")
    d = draw(g, "infer", 42)
    with forced(1, plan):
        y = H.gpu_conv_bias(g, d["x"], d["w"], d["bias"], True)
    H.assert_close(y, H.oracle.conv2d_bias_act(H.oshape(g), d["x"], d["w"], d["bias"], True), "conv+bias+relu")


@pytest.mark.parametrize("stage", [2, 3, 4], ids=["dgrad", "wgrad", "schedule"])
# + a stride-2 layer (no data gradient) and a layer whose generic weight gradient splits
# the pixels more finely (15 splits) than the transposed-read one (12): the fused schedule
# runs the generic kernel, so the workspace must hold its partials.
# Two more layers for the 256 x 256 transposed-read weight gradient (C % 256 == 0): two
# output-channel tiles with a ragged last pixel split, and a 1x1 layer with two taps'
# worth of channels per tile row.  For the x-row offsets the transposed-read weight
# gradient steps by 64 pixels per slice (row and image wraps): a vertical stride of 2 with
# a 1x3 filter, and 5x3 images, where a step of 64 pixels crosses several images.
@pytest.mark.parametrize("g", PLAN_GEOMS[:4] + [Geometry(2, 17, 13, 64, 64, 3, 3, 2, 1),
                                                Geometry(30, 8, 16, 256, 256, 3, 3, 1, 1),
                                                Geometry(7, 9, 11, 256, 512, 3, 3, 1, 1),
                                                Geometry(3, 10, 10, 512, 256, 1, 1, 1, 0),
                                                Geometry(3, 11, 9, 128, 256, 1, 3, 2, 0, stride_w=1, pad_w=1),
                                                Geometry(5, 5, 3, 128, 256, 3, 3, 1, 1)], ids=str)
def test_backward_plans(g, stage):
    want_dx = g.sh == 1 and g.sw == 1
    if stage == 2 and not want_dx:
        pytest.skip("the data gradient needs stride 1")
    d = draw(g, "bwd", 43)
    res, devt = H.gpu_train(g, d)
    ob = H.oracle_backward_on_gpu_state(g, d, res, d["dy"], want_dx=want_dx)
    ref = H.gpu_backward(g, devt, d["dy"], want_dx=want_dx)
    for plan in eligible(g, stage):
        H.log(f"stage {stage} plan {lib().cbr_plan_name(plan).decode()} {g}")
        with forced(stage, plan):
            bw = H.gpu_backward(g, devt, d["dy"], want_dx=want_dx)
        H.check_backward(g, d, bw, ob, want_dx)
        if stage == 4:
            # without a dz output (the fused schedule forms dz inside the gradients, with
            # the apply kernel's arithmetic, so the dz the gradients read is the one the
            # default schedule stores)
            with forced(stage, plan):
                bn = H.gpu_backward(g, devt, d["dy"], want_dx=want_dx, dz_out=False)
            for k in ("dgamma", "dbeta"):
                np.testing.assert_array_equal(bn[k], ref[k], err_msg=k)
            H.check_backward(g, d, dict(bn, dz=ref["dz"]), ob, want_dx)
