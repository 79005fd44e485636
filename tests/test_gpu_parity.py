"""GPU parity: the HIP library, called through its C ABI, against the fp64 oracle on
the same seeded inputs, element by element (tolerances in tests/cbr_harness.py)."""
import numpy as np
import pytest

from conv2d_batchnorm_relu_amd.inputs import Geometry, draw, draw_workload, WORKLOADS
import cbr_harness as H

pytestmark = pytest.mark.gpu

# Small geometries that still span several tiles and ragged tails (tiles are 128 output
# pixels x 64 or 128 output channels; K-steps are 64 reduction elements).
TRAIN_GEOMS = [
    Geometry(2, 8, 8, 4, 8, 3, 3, 1, 1),         # the tiny workload (C=4: scalar gather path)
    Geometry(3, 9, 11, 16, 24, 3, 3, 1, 1),      # ragged M (297), K=24 < one channel tile
    Geometry(2, 17, 13, 64, 64, 3, 3, 2, 1),     # stride 2
    Geometry(2, 31, 29, 3, 64, 7, 7, 2, 3),      # first-layer form: Cin=3, 7x7, stride 2
    Geometry(1, 12, 12, 128, 128, 3, 3, 1, 1),   # K=128 tile, Kg=1152
    Geometry(2, 7, 9, 256, 256, 3, 3, 1, 1),     # two channel tiles
    Geometry(4, 14, 14, 64, 72, 1, 1, 1, 0),     # 1x1, K=72 (ragged channel tile)
    Geometry(2, 10, 10, 8, 16, 3, 3, 1, 1),      # C=8: K-steps span several taps
    Geometry(1, 1, 2, 8, 8, 1, 1, 1, 0),         # two output pixels (the fewest training allows)
]
INFER_GEOMS = TRAIN_GEOMS + [Geometry(1, 1, 1, 8, 8, 1, 1, 1, 0)]   # a single output pixel


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import conv2d_batchnorm_relu_amd as cbr
    cbr._load()


@pytest.mark.parametrize("g", TRAIN_GEOMS, ids=str)
def test_train_forward_small(g):
    H.log(f"train fwd {g}")
    d = draw(g, "train", 7)
    res, _ = H.gpu_train(g, d)
    ora = H.oracle_train(g, d)
    H.check_train(g, d, res, ora)


# The persistent 3x3 / 64-channel kernel (W a multiple of 8, 8..56; steps of 256 pixels
# that start anywhere in a row; each workgroup a contiguous range of the batch's steps):
# partial last steps and pixel blocks, steps spanning up to 33 rows, ranges that start
# inside an image (batches of fewer steps than workgroups) and that cross image ends
# (N > 256), images smaller than one step.
# The 64-channel 3x3 shapes it does not take (W % 8 != 0) run the generic conv.
HALO_GEOMS = [
    Geometry(2, 12, 16, 64, 64, 3, 3, 1, 1),     # one step of 6 blocks
    Geometry(3, 9, 24, 64, 64, 3, 3, 1, 1),      # one step of 6.75 blocks
    Geometry(1, 56, 56, 64, 64, 3, 3, 1, 1),     # one full image, thirteen steps
    Geometry(300, 5, 8, 64, 64, 3, 3, 1, 1),     # two images for some workgroups
    Geometry(2, 3, 56, 64, 64, 3, 3, 1, 1),      # fewer pixels than a step
    Geometry(2, 17, 8, 64, 64, 3, 3, 1, 1),      # the narrowest image
    Geometry(1, 6, 40, 64, 64, 3, 3, 1, 1),      # 7.5 blocks
    Geometry(2, 7, 48, 64, 64, 3, 3, 1, 1),      # a full step, then 2.5 blocks
    Geometry(2, 29, 56, 64, 64, 3, 3, 1, 1),     # steps starting mid-row, a 1/3 last step
    Geometry(1, 40, 24, 64, 64, 3, 3, 1, 1),     # 3.75 steps of up to 12 rows
    Geometry(1, 70, 8, 64, 64, 3, 3, 1, 1),      # steps of 32 rows
    Geometry(300, 9, 32, 64, 64, 3, 3, 1, 1),    # a step and a block per image, N > 256
    Geometry(2, 12, 12, 64, 64, 3, 3, 1, 1),     # generic conv (W % 8 != 0)
    Geometry(300, 5, 7, 64, 64, 3, 3, 1, 1),     # generic conv, N > 256
]


@pytest.mark.parametrize("n", [32, 300])
def test_train_forward_headline_shape_other_batches(n):
    """The persistent 3x3 kernel on the 56x56x64 layer at N = 32 (256 ranges of one or two
    steps, most starting inside an image) and N = 300 (ranges crossing image ends), forced
    whatever the plan table prefers, every output against the oracle."""
    import ctypes
    import conv2d_batchnorm_relu_amd as cbr
    wl, d = draw_workload("s2_train", n=n)
    g = wl.geom
    lib = cbr._load()
    assert lib.cbr_set_plan_override(0, 1) == 0
    try:
        assert lib.cbr_plan_of(ctypes.byref(H.cshape(g)), 0) == 1
        H.log(f"persistent 3x3, N = {n}")
        res, _ = H.gpu_train(g, d, wl.eps, wl.momentum)
    finally:
        lib.cbr_set_plan_override(0, 0)
    ora = H.oracle_train(g, d, wl.eps, wl.momentum)
    H.check_train(g, d, res, ora, wl.eps, wl.momentum)


@pytest.mark.parametrize("g", HALO_GEOMS, ids=str)
def test_train_forward_persistent_3x3(g):
    H.log(f"train fwd (persistent 3x3) {g}")
    d = draw(g, "train", 14)
    res, _ = H.gpu_train(g, d)
    ora = H.oracle_train(g, d)
    H.check_train(g, d, res, ora)


# The first-layer kernel (3 input channels, stride 2, 64 output channels, W % 8 == 0;
# persistent over ranges of 256-pixel steps): partial last steps, short and narrow images,
# 3x3, 5x5 and non-square filters, ranges starting inside an image and crossing image
# ends, one 8-pixel piece per input row.
FIRST_LAYER_GEOMS = [
    Geometry(2, 32, 32, 3, 64, 7, 7, 2, 3),
    Geometry(1, 24, 40, 3, 64, 7, 7, 2, 3),
    Geometry(3, 17, 16, 3, 64, 3, 3, 2, 1),      # 9 x 8 outputs: one partial step per image
    Geometry(2, 40, 8, 3, 64, 5, 5, 2, 1),       # 3 output columns
    Geometry(1, 224, 224, 3, 64, 7, 7, 2, 3),    # one image: 49 single-step ranges, most mid-image
    Geometry(300, 16, 16, 3, 64, 3, 3, 2, 1),    # 300 one-step images over 256 workgroups
    Geometry(3, 9, 8, 3, 64, 3, 6, 2, 1, pad_w=0),   # two output columns, one 8-pixel piece per row
    Geometry(2, 31, 24, 3, 64, 4, 6, 2, 2),      # even padding, R != S
    Geometry(4, 64, 64, 3, 64, 1, 1, 2, 0),      # a 1 x 1 filter: one k-step per chain
    Geometry(2, 50, 40, 3, 64, 2, 2, 2, 0),      # R = 2, no padding
    Geometry(5, 30, 24, 3, 64, 6, 4, 2, 2, pad_w=1),   # R = 6, padding (2, 1)
    Geometry(3, 12, 8, 3, 64, 6, 6, 2, 2),       # one 24-pixel step per image, R = 6
    Geometry(1, 300, 296, 3, 64, 7, 7, 2, 3),    # 150 output columns, 302-pixel ring rows
]


@pytest.mark.parametrize("g", FIRST_LAYER_GEOMS, ids=str)
def test_train_forward_first_layer(g):
    H.log(f"train fwd (first layer) {g}")
    d = draw(g, "train", 15)
    res, _ = H.gpu_train(g, d)
    ora = H.oracle_train(g, d)
    H.check_train(g, d, res, ora)


# The persistent large-tile conv (C % 32 == 0, K a multiple of 128; at most 256
# workgroups over contiguous pixel ranges).  K = 256 with at most 224 pixels per
# workgroup runs one 224 x 256 chunk per workgroup; everything else 448 x 128 chunks:
# several chunks per workgroup, a short last chunk, several channel chunks, 1x1 / 5x5 /
# stride 2, C = 96 (32-element slices).
IGEMM_TRAIN_GEOMS = [
    Geometry(3, 13, 11, 64, 256, 3, 3, 1, 1),      # ragged ranges: 31 pixels per workgroup
    Geometry(256, 10, 20, 32, 256, 1, 1, 1, 0),    # 200 pixels per workgroup, one slice
    Geometry(16, 14, 14, 96, 256, 3, 3, 2, 1),     # stride 2, three slices per tap
]
IGEMM_INFER_GEOMS = IGEMM_TRAIN_GEOMS + [
    Geometry(3, 160, 160, 32, 128, 3, 3, 1, 1),    # 300 pixels per workgroup: chunks of 256 and 44
    Geometry(2, 200, 160, 32, 256, 1, 1, 1, 0),    # 250 per workgroup: 256 x 128 chunks, two channel chunks
    Geometry(2, 99, 101, 64, 128, 3, 3, 2, 1),     # stride 2, padding on every side
    Geometry(2, 19, 23, 32, 128, 5, 5, 1, 2),      # 5x5
    Geometry(4, 14, 14, 64, 384, 1, 1, 1, 0),      # three channel chunks
]


@pytest.mark.parametrize("g", IGEMM_TRAIN_GEOMS, ids=str)
def test_train_forward_large_tile(g):
    H.log(f"train fwd (large-tile conv) {g}")
    d = draw(g, "train", 17)
    res, _ = H.gpu_train(g, d)
    ora = H.oracle_train(g, d)
    H.check_train(g, d, res, ora)


@pytest.mark.parametrize("g", IGEMM_INFER_GEOMS, ids=str)
def test_infer_large_tile(g):
    H.log(f"infer (large-tile conv) {g}")
    d = draw(g, "infer", 18)
    y = H.gpu_infer(g, d)
    ref = H.oracle.forward_infer(H.oshape(g), d["x"], d["w"], d["bias"], d["gamma"], d["beta"],
                                 d["run_mean"], d["run_var"], 1e-5)
    H.assert_close(y, ref, "infer y")


@pytest.mark.parametrize("g", INFER_GEOMS, ids=str)
def test_infer_small(g):
    H.log(f"infer {g}")
    d = draw(g, "infer", 8)
    y = H.gpu_infer(g, d)
    ref = H.oracle.forward_infer(H.oshape(g), d["x"], d["w"], d["bias"], d["gamma"], d["beta"],
                                 d["run_mean"], d["run_var"], 1e-5)
    H.assert_close(y, ref, "infer y")


def test_infer_without_bias():
    g = Geometry(2, 9, 9, 32, 32, 3, 3, 1, 1)
    d = draw(g, "infer", 9)
    d["bias"] = None
    y = H.gpu_infer(g, d)
    ref = H.oracle.forward_infer(H.oshape(g), d["x"], d["w"], None, d["gamma"], d["beta"],
                                 d["run_mean"], d["run_var"], 1e-5)
    H.assert_close(y, ref, "infer y (no bias)")


BWD_GEOMS = [
    (Geometry(2, 8, 8, 4, 8, 3, 3, 1, 1), True),       # tiny: C=4 dgrad output (scalar stores)
    (Geometry(3, 9, 11, 16, 24, 3, 3, 1, 1), True),
    (Geometry(2, 7, 9, 256, 256, 3, 3, 1, 1), True),
    (Geometry(2, 12, 12, 64, 64, 3, 3, 1, 1), True),
    (Geometry(2, 17, 13, 64, 64, 3, 3, 2, 1), False),  # stride 2: first-layer form, no dx
    (Geometry(2, 31, 29, 3, 64, 7, 7, 2, 3), False),   # Cin=3 7x7 s2 weight gradient
    (Geometry(4, 14, 14, 64, 72, 1, 1, 1, 0), True),
    (Geometry(2, 12, 12, 128, 128, 3, 3, 1, 1), True),   # data gradient on 256 x 128 chunks
    (Geometry(3, 13, 11, 256, 64, 3, 3, 1, 1), True),    # data gradient: 64 -> 256 channels
    (Geometry(2, 9, 11, 128, 512, 3, 3, 2, 1), False),   # transposed-read weight gradient: 2 x 9 tiles, stride 2
    (Geometry(5, 12, 12, 128, 256, 1, 1, 1, 0), True),   # transposed-read weight gradient, 1x1, ragged pixel split
    (Geometry(4, 48, 47, 128, 256, 3, 3, 1, 1), False),  # 6 slices per split, a 3-slice last split
]


@pytest.mark.parametrize("g,want_dx", BWD_GEOMS, ids=str)
def test_backward_small(g, want_dx):
    H.log(f"backward {g} dx={want_dx}")
    d = draw(g, "bwd", 10)
    res, devt = H.gpu_train(g, d)
    bw = H.gpu_backward(g, devt, d["dy"], want_dx=want_dx)
    ob = H.oracle_backward_on_gpu_state(g, d, res, d["dy"], want_dx=want_dx)
    H.check_backward(g, d, bw, ob, want_dx)
    if not want_dx:
        assert bw["dx"] is None


# Anisotropic geometry (stride, padding and filter size differ between the axes) through
# every kernel family that accepts it: the generic conv, the large-tile conv, the
# first-layer conv, both weight-gradient kernels and the data gradient.
ANISO_TRAIN_GEOMS = [
    Geometry(3, 9, 11, 16, 24, 3, 5, stride=2, pad=1, stride_w=1, pad_w=2),    # generic conv
    Geometry(2, 13, 10, 8, 16, 7, 1, stride=1, pad=3, stride_w=2, pad_w=0),    # generic conv, 7x1
    Geometry(3, 13, 11, 64, 256, 3, 5, stride=2, pad=1, stride_w=1, pad_w=2),  # large-tile conv
    Geometry(2, 11, 15, 32, 128, 1, 3, stride=1, pad=0, stride_w=2, pad_w=1),  # large-tile conv, 1x3
    Geometry(2, 32, 32, 3, 64, 7, 5, stride=2, pad=2, pad_w=1),                # first layer, 7x5
    Geometry(2, 30, 24, 3, 64, 5, 7, stride=2, pad=1, pad_w=3),                # first layer, 5x7
]
ANISO_INFER_GEOMS = ANISO_TRAIN_GEOMS[:4] + [
    Geometry(2, 19, 23, 32, 128, 7, 1, stride=1, pad=3, stride_w=2, pad_w=0),  # large-tile conv, 7x1
]
ANISO_BWD_GEOMS = [
    (Geometry(2, 9, 11, 16, 24, 3, 5, stride=1, pad=1, pad_w=2), True),        # generic wgrad + dgrad
    (Geometry(2, 10, 12, 128, 256, 3, 1, stride=1, pad=1, pad_w=0), True),     # transposed-read wgrad, large-tile dgrad
    (Geometry(2, 13, 9, 128, 256, 3, 3, stride=2, pad=1, stride_w=1), False),  # transposed-read wgrad, stride (2,1)
    (Geometry(3, 12, 10, 16, 32, 1, 3, stride=1, pad=0, stride_w=2, pad_w=1), False),  # generic wgrad, stride (1,2)
    (Geometry(2, 31, 29, 3, 64, 7, 5, stride=2, pad=3, pad_w=1), False),       # first-layer wgrad, 7x5
]


@pytest.mark.parametrize("g", ANISO_TRAIN_GEOMS, ids=str)
def test_train_forward_anisotropic(g):
    H.log(f"train fwd (anisotropic) {g}")
    d = draw(g, "train", 19)
    res, _ = H.gpu_train(g, d)
    ora = H.oracle_train(g, d)
    H.check_train(g, d, res, ora)


@pytest.mark.parametrize("g", ANISO_INFER_GEOMS, ids=str)
def test_infer_anisotropic(g):
    H.log(f"infer (anisotropic) {g}")
    d = draw(g, "infer", 20)
    y = H.gpu_infer(g, d)
    ref = H.oracle.forward_infer(H.oshape(g), d["x"], d["w"], d["bias"], d["gamma"], d["beta"],
                                 d["run_mean"], d["run_var"], 1e-5)
    H.assert_close(y, ref, "infer y")


@pytest.mark.parametrize("g,want_dx", ANISO_BWD_GEOMS, ids=str)
def test_backward_anisotropic(g, want_dx):
    H.log(f"backward (anisotropic) {g} dx={want_dx}")
    d = draw(g, "bwd", 21)
    res, devt = H.gpu_train(g, d)
    bw = H.gpu_backward(g, devt, d["dy"], want_dx=want_dx)
    ob = H.oracle_backward_on_gpu_state(g, d, res, d["dy"], want_dx=want_dx)
    H.check_backward(g, d, bw, ob, want_dx)


# Channels whose batch mean is many standard deviations from zero: input channel 0 is the
# constant 1 and the centre tap of each filter scales it, so every output pixel sees it
# (the centre tap is never in the padding) and output channel k gets mean ~ +-ratio*sigma_k,
# sigma_k the spread the other channels give it.  One geometry per statistics kernel.
LARGE_MEAN_GEOMS = [
    Geometry(2, 12, 16, 64, 64, 3, 3, 1, 1),       # persistent 3x3 conv
    Geometry(3, 13, 11, 64, 256, 3, 3, 1, 1),      # large-tile conv
    Geometry(3, 9, 11, 16, 24, 3, 3, 1, 1),        # generic conv
    Geometry(2, 32, 32, 3, 64, 7, 7, 2, 3),        # first-layer conv
]


def large_mean_inputs(g, ratio, seed):
    from conv2d_batchnorm_relu_amd.inputs import bf16_round
    d = draw(g, "train", seed)
    x = d["x"].copy()
    x[..., 0] = 1.0
    w = d["w"].copy()
    w[:, g.r // 2, g.s // 2, 0] = 0.0
    sigma = np.sqrt((w.astype(np.float64) ** 2).reshape(g.k, -1).sum(1))
    sign = np.where(np.arange(g.k) % 2 == 0, 1.0, -1.0)
    w[:, g.r // 2, g.s // 2, 0] = (sign * ratio * sigma).astype(np.float32)
    d["x"], d["w"] = bf16_round(x), bf16_round(w)
    return d


@pytest.mark.parametrize("ratio", [10.0, 100.0])
@pytest.mark.parametrize("g", LARGE_MEAN_GEOMS, ids=str)
def test_train_forward_large_channel_mean(g, ratio):
    H.log(f"train fwd (|mean|/sigma ~ {ratio}) {g}")
    d = large_mean_inputs(g, ratio, 22)
    res, _ = H.gpu_train(g, d)
    ora = H.oracle_train(g, d)
    got = np.abs(ora["mean"]) / np.sqrt(ora["var"])
    assert got.min() > 0.5 * ratio, got.min()
    # y and the mask are compared with the normalisation of the stored bf16 z: at these
    # ratios the rounding of z to bf16 alone moves u by up to ratio * 2^-9 * gamma.
    H.check_train(g, d, res, ora, y_from_stored_z=True)


# Conv2D + bias (+ ReLU) without batch normalisation: the generic conv (small and ragged
# channel counts, anisotropic geometry) and the large-tile conv, with and without bias.
CONV_BIAS_GEOMS = [
    Geometry(3, 9, 11, 16, 24, 3, 3, 1, 1),
    Geometry(2, 13, 10, 8, 16, 7, 1, stride=1, pad=3, stride_w=2, pad_w=0),
    Geometry(2, 17, 13, 64, 64, 3, 3, 2, 1),
    Geometry(3, 13, 11, 64, 256, 3, 3, 1, 1),          # large-tile conv, 224 x 256 chunks
    Geometry(3, 160, 160, 32, 128, 3, 3, 1, 1),        # large-tile conv, 448 x 128 chunks
    Geometry(2, 11, 15, 32, 128, 1, 3, stride=1, pad=0, stride_w=2, pad_w=1),
]


@pytest.mark.parametrize("relu", [True, False], ids=["relu", "linear"])
@pytest.mark.parametrize("with_bias", [True, False], ids=["bias", "nobias"])
@pytest.mark.parametrize("g", CONV_BIAS_GEOMS, ids=str)
def test_conv_bias_act(g, with_bias, relu):
    H.log(f"conv + bias (relu={relu}, bias={with_bias}) {g}")
    d = draw(g, "infer", 23)
    bias = d["bias"] if with_bias else None
    y = H.gpu_conv_bias(g, d["x"], d["w"], bias, relu)
    ref = H.oracle.conv2d_bias_act(H.oshape(g), d["x"], d["w"], bias, relu)
    H.assert_close(y, ref, "conv + bias" + (" + relu" if relu else ""))
    if not relu:
        assert (y < 0).any()


def test_conv_bias_relu_full_size():
    """The 28x28x128 layer (N = 256, 3x3, bias) that the benchmark times, every output."""
    g = Geometry(256, 28, 28, 128, 128, 3, 3, 1, 1)
    d = draw(g, "infer", 24)
    H.log(f"conv + bias + relu, full size {g}")
    y = H.gpu_conv_bias(g, d["x"], d["w"], d["bias"], True)
    ref = H.oracle.conv2d_bias_act(H.oshape(g), d["x"], d["w"], d["bias"], True)
    H.assert_close(y, ref, "conv + bias + relu")


def test_backward_dz_in_workspace_and_dx_aliasing_x():
    """dz = NULL keeps dz in the workspace; dx may overwrite x in place."""
    g = Geometry(2, 12, 12, 32, 32, 3, 3, 1, 1)
    d = draw(g, "bwd", 11)
    res, devt = H.gpu_train(g, d)
    ref = H.gpu_backward(g, devt, d["dy"])
    alias = H.gpu_backward(g, devt, d["dy"], dz_out=False, dx_alias_x=True)
    for k in ("dgamma", "dbeta", "dw", "dx"):
        np.testing.assert_array_equal(alias[k], ref[k], err_msg=k)


def test_running_stats_in_place():
    g = Geometry(2, 9, 9, 16, 16, 3, 3, 1, 1)
    d = draw(g, "train", 12)
    d["run_mean"] = np.linspace(-1, 1, g.k).astype(np.float32)
    d["run_var"] = np.linspace(0.5, 2, g.k).astype(np.float32)
    res, _ = H.gpu_train(g, d, inplace_running=True)
    ora = H.oracle_train(g, d)
    H.check_train(g, d, res, ora)


def test_bitwise_deterministic():
    g = Geometry(8, 20, 24, 64, 64, 3, 3, 1, 1)
    d = draw(g, "bwd", 13)
    r1, dv1 = H.gpu_train(g, d)
    r2, dv2 = H.gpu_train(g, d)
    for k in ("z", "y", "mask_words", "mean", "invstd", "run_mean", "run_var"):
        np.testing.assert_array_equal(r1[k], r2[k], err_msg=k)
    b1 = H.gpu_backward(g, dv1, d["dy"])
    b2 = H.gpu_backward(g, dv2, d["dy"])
    for k in b1:
        np.testing.assert_array_equal(b1[k], b2[k], err_msg=k)


# ----------------------------------------------------------------------------------
# full-size workloads, complete outputs against the complete oracle
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "stem", "s2_train"])
def test_train_full_workload(name):
    wl, d = draw_workload(name)
    g = wl.geom
    if not wl.bf16:   # the fp32 workload runs on the bf16 path with its values pre-rounded
        from conv2d_batchnorm_relu_amd.inputs import bf16_round
        d = {k: (bf16_round(v) if k in ("x", "w", "dy") else v) for k, v in d.items()}
    H.log(f"full train {name} {g}")
    res, devt = H.gpu_train(g, d, wl.eps, wl.momentum)
    H.log("oracle")
    ora = H.oracle_train(g, d, wl.eps, wl.momentum)
    flips = H.check_train(g, d, res, ora, wl.eps, wl.momentum)
    H.log(f"ok, mask flips near zero: {flips}")
    if name == "tiny":
        bw = H.gpu_backward(g, devt, d["dy"])
        ob = H.oracle_backward_on_gpu_state(g, d, res, d["dy"])
        H.check_backward(g, d, bw, ob)


def test_infer_full_workload():
    wl, d = draw_workload("s3_infer")
    g = wl.geom
    H.log(f"full infer {g}")
    y = H.gpu_infer(g, d, wl.eps)
    ref = H.oracle.forward_infer(H.oshape(g), d["x"], d["w"], d["bias"], d["gamma"], d["beta"],
                                 d["run_mean"], d["run_var"], wl.eps)
    H.assert_close(y, ref, "infer y")


def test_backward_full_workload():
    wl, d = draw_workload("s4_bwd")
    g = wl.geom
    H.log(f"full backward {g}")
    res, devt = H.gpu_train(g, d, wl.eps, wl.momentum)
    bw = H.gpu_backward(g, devt, d["dy"])
    H.log("oracle forward")
    ora = H.oracle_train(g, d, wl.eps, wl.momentum)
    flips = H.check_train(g, d, res, ora, wl.eps, wl.momentum)
    H.log(f"forward ok, mask flips near zero: {flips}; oracle backward")
    ob = H.oracle_backward_on_gpu_state(g, d, res, d["dy"])
    H.check_backward(g, d, bw, ob)


@pytest.mark.parametrize("g", [Geometry(2, 6, 10, 8, 8, 1, 1, 1, 0),        # generic kernel
                               Geometry(2, 6, 16, 64, 64, 3, 3, 1, 1)],     # persistent 3x3 kernel
                         ids=["generic", "persistent3x3"])
def test_z_rounding_is_nearest_even(g):
    """z = x0 + x1 with x0 = 1 + j*2^-7 and x1 in {2^-8, 3*2^-8, 2^-9}: exact fp32 sums that sit
    on (or next to) bf16 rounding ties; the stored z must be their round-to-nearest-even."""
    from conv2d_batchnorm_relu_amd.inputs import bf16_round
    rng = np.random.default_rng(15)
    x = np.zeros((g.n, g.h, g.w, g.c), np.float32)
    x[..., 0] = 1.0 + rng.integers(0, 8, (g.n, g.h, g.w)) * 2.0 ** -7
    x[..., 1] = rng.choice(np.array([2.0 ** -8, 3 * 2.0 ** -8, 2.0 ** -9], np.float32), (g.n, g.h, g.w))
    w = np.zeros((g.k, g.r, g.s, g.c), np.float32)
    w[:, g.r // 2, g.s // 2, 0] = 1.0
    w[:, g.r // 2, g.s // 2, 1] = 1.0
    d = draw(g, "train", 16)
    d["x"], d["w"] = x, w
    res, _ = H.gpu_train(g, d)
    exact = (x[..., 0] + x[..., 1]).astype(np.float32)              # exact in fp32
    want = np.broadcast_to(bf16_round(exact)[..., None], res["z"].shape)
    np.testing.assert_array_equal(res["z"], want)
    assert (bf16_round(exact) != exact).any()                         # ties were really exercised
