"""Host-side checks of the C ABI: the library loads, exports every function that
include/cbr.h declares, and its validation rejects bad arguments before any HIP call.
Every call here fails validation on purpose (fake pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

import conv2d_batchnorm_relu_amd as cbr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cbr.h")

FAKE = 0x100000  # 16-byte-aligned fake device address (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(cbr.library_path()):
        pytest.fail("libcbr.so is not built; run __graft_entry__.build()")
    return cbr._load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cbr_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"cbr_forward_train", "cbr_forward_infer", "cbr_backward", "cbr_workspace_bytes"} <= set(names)
    raw = ctypes.CDLL(cbr.library_path())
    for n in names:
        assert hasattr(raw, n), f"{n} declared in cbr.h but not exported"


def test_status_strings(lib):
    for s in range(8):
        assert cbr.cbr_status_str(s).startswith("CBR")
    assert "unknown" in cbr.cbr_status_str(99)


def shp(**kw):
    base = dict(n=2, h=8, w=8, c=4, k=8, r=3, s=3, stride=1, pad=1)
    base.update(kw)
    return cbr.make_shape(**base)


def test_output_hw_and_mask_words(lib):
    assert cbr.cbr_output_hw(shp()) == (8, 8)
    assert cbr.cbr_output_hw(shp(n=64, h=224, w=224, c=3, k=64, r=7, s=7, stride=2, pad=3)) == (112, 112)
    assert cbr.cbr_output_hw(shp(h=7, w=6, r=3, s=3, stride=2, pad=0)) == (3, 2)
    assert cbr.cbr_mask_words(shp()) == 2 * 8 * 8 * 8 // 32
    assert cbr.cbr_mask_words(shp(n=1, h=1, w=1, c=8, k=8, r=1, s=1, pad=0)) == 1   # 8 bits -> 1 word


@pytest.mark.parametrize("kw,status", [
    (dict(n=0), 2), (dict(h=-1), 2), (dict(stride=0), 2), (dict(pad=-1), 2),
    (dict(h=2, r=7, s=7, pad=2), 2),            # filter larger than the padded input
    (dict(k=12), 3), (dict(k=4096), 3),          # K % 8, K > 2048
    (dict(pad=3), 3),                            # pad >= filter size
    (dict(n=70000, h=200, w=200, c=64), 3),      # tensor of 2^31 elements or more
    (dict(n=300, h=256, w=256, c=64), 3),        # 2^30 elements or more (byte offsets need 31 bits)
])
def test_shape_validation(lib, kw, status):
    with pytest.raises(cbr.CbrError) as e:
        cbr.cbr_output_hw(shp(**kw))
    assert e.value.status == status
    assert cbr.cbr_workspace_bytes(shp(**kw), cbr.CBR_OP_TRAIN) == 0


def test_workspace_sizes_positive_and_monotone(lib):
    small = cbr.cbr_workspace_bytes(shp(), cbr.CBR_OP_TRAIN)
    big = cbr.cbr_workspace_bytes(shp(n=64), cbr.CBR_OP_TRAIN)
    assert 0 < small <= big
    for op in (0, 1, 2):
        assert cbr.cbr_workspace_bytes(shp(), op) % 256 == 0
    assert cbr.cbr_workspace_bytes(shp(), 7) == 0


def _train(sp, **over):
    a = dict(x=FAKE, w=FAKE, gamma=FAKE, beta=FAKE, rm=FAKE, rv=FAKE, eps=1e-5, mom=0.1, z=FAKE, y=FAKE,
             mask=FAKE, sm=FAKE, si=FAKE, rmo=FAKE, rvo=FAKE, ws=FAKE, nbytes=1 << 30)
    a.update(over)
    return cbr._load().cbr_forward_train(ctypes.byref(sp), a["x"], a["w"], a["gamma"], a["beta"], a["rm"],
                                         a["rv"], a["eps"], a["mom"], a["z"], a["y"], a["mask"], a["sm"],
                                         a["si"], a["rmo"], a["rvo"], a["ws"], a["nbytes"], 0)


@pytest.mark.parametrize("over,status", [
    (dict(x=None), 1), (dict(mask=None), 1), (dict(rvo=None), 1),
    (dict(y=FAKE + 2), 4), (dict(gamma=FAKE + 4), 4),
    (dict(ws=None), 5), (dict(nbytes=16), 5),
    (dict(eps=-1.0), 7), (dict(mom=1.5), 7), (dict(eps=float("inf")), 7), (dict(mom=float("nan")), 7),
])
def test_train_validation(lib, over, status):
    assert _train(shp(), **over) == status


def test_training_needs_two_output_pixels(lib):
    one = shp(n=1, h=1, w=1, c=8, k=8, r=1, s=1, pad=0)
    assert cbr.cbr_output_hw(one) == (1, 1)          # a valid shape ...
    assert _train(one) == 2                           # ... but no batch variance from one value
    assert _bwd(one) == 2


def test_train_null_shape(lib):
    st = cbr._load().cbr_forward_train(None, *([FAKE] * 6), 1e-5, 0.1, *([FAKE] * 8), 1 << 30, 0)
    assert st == 1


def _bwd(sp, **over):
    a = dict(x=FAKE, w=FAKE, z=FAKE, mask=FAKE, dy=FAKE, gamma=FAKE, sm=FAKE, si=FAKE, dz=FAKE, dg=FAKE,
             db=FAKE, dw=FAKE, dx=FAKE, ws=FAKE, nbytes=1 << 30)
    a.update(over)
    return cbr._load().cbr_backward(ctypes.byref(sp), a["x"], a["w"], a["z"], a["mask"], a["dy"], a["gamma"],
                                    a["sm"], a["si"], a["dz"], a["dg"], a["db"], a["dw"], a["dx"], a["ws"],
                                    a["nbytes"], 0)


@pytest.mark.parametrize("over,status", [
    (dict(dy=None), 1), (dict(dw=None), 1), (dict(dx=FAKE + 8), 4), (dict(dz=FAKE + 8), 4),
    (dict(nbytes=0), 5),
])
def test_backward_validation(lib, over, status):
    assert _bwd(shp(), **over) == status


def test_backward_dx_needs_stride_one(lib):
    assert _bwd(shp(stride=2)) == 3


def _infer(sp, **over):
    a = dict(x=FAKE, w=FAKE, bias=None, gamma=FAKE, beta=FAKE, rm=FAKE, rv=FAKE, eps=1e-5, y=FAKE, ws=FAKE,
             nbytes=1 << 30)
    a.update(over)
    return cbr._load().cbr_forward_infer(ctypes.byref(sp), a["x"], a["w"], a["bias"], a["gamma"], a["beta"],
                                         a["rm"], a["rv"], a["eps"], a["y"], a["ws"], a["nbytes"], 0)


@pytest.mark.parametrize("over,status", [
    (dict(y=None), 1), (dict(bias=FAKE + 4), 4), (dict(ws=FAKE + 8), 4), (dict(nbytes=1), 5),
    (dict(eps=-0.5), 7),
])
def test_infer_validation(lib, over, status):
    assert _infer(shp(), **over) == status


@pytest.mark.parametrize("name", ["cbr_conv2d_bias_relu", "cbr_conv2d_bias"])
@pytest.mark.parametrize("args,status", [
    ((None, FAKE, FAKE, FAKE), 1), ((FAKE, FAKE, None, None), 1), ((FAKE, FAKE, FAKE + 4, FAKE), 4),
    ((FAKE + 2, FAKE, None, FAKE), 4),
])
def test_conv_bias_validation(lib, name, args, status):
    x, w, b, y = args
    assert getattr(cbr._load(), name)(ctypes.byref(shp()), x, w, b, y, 0) == status
    assert getattr(cbr._load(), name)(ctypes.byref(shp(k=12)), FAKE, FAKE, None, FAKE, 0) == 3


def test_product_never_imports_oracle():
    """The package and the library sources do not reference the oracle."""
    pkg = os.path.join(ROOT, "conv2d_batchnorm_relu_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower() or f == "inputs.py", f
                assert "cbro_" not in text, f


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(cbr, "_LIB_PATH", str(tmp_path / "libcbr.so"))
    monkeypatch.setattr(cbr, "_lib", None)
    with pytest.raises(ImportError):
        cbr.cbr_status_str(0)


def test_binding_rejects_unusable_tensors():
    """The binding refuses host tensors, non-contiguous views and wrong element sizes
    before anything reaches the library (it never reinterprets memory)."""
    import torch
    import conv2d_batchnorm_relu_amd as cbr
    sp = cbr.make_shape(1, 4, 4, 8, 8, 3, 3, 1, 1)
    host = torch.zeros(16, dtype=torch.bfloat16)
    args = [host] * 6 + [1e-5, 0.1] + [host] * 8 + [None]
    with pytest.raises(cbr.CbrError, match="not a GPU tensor"):
        cbr.cbr_forward_train(sp, *args)
    with pytest.raises(cbr.CbrError, match="not a GPU tensor"):
        cbr.cbr_forward_infer(sp, host, host, None, host, host, host, host, 1e-5, host, None)
    with pytest.raises(cbr.CbrError, match="not a GPU tensor"):
        cbr.cbr_backward(sp, host, host, host, host, host, host, host, host, None, host, host, host, None, None)


def test_noalloc_rejects_shapes_beyond_its_scratch(lib):
    """The allocation-free training forward refuses, before touching the GPU, a shape whose
    scratch needs exceed its fixed array; shape errors keep their own codes."""
    big = cbr.make_shape(4096, 56, 56, 64, 72, 3, 3, 1, 1)   # generic conv: ~100k statistics rows
    assert cbr.cbr_workspace_bytes(big, cbr.CBR_OP_TRAIN) > 4 << 20
    fn = cbr._load().cbr_forward_train_noalloc
    assert fn(ctypes.byref(big), *([FAKE] * 6), 1e-5, 0.1, *([FAKE] * 8), 0) == 5      # CBR_E_WORKSPACE
    assert fn(ctypes.byref(shp(k=12)), *([FAKE] * 6), 1e-5, 0.1, *([FAKE] * 8), 0) == 3
    assert fn(None, *([FAKE] * 6), 1e-5, 0.1, *([FAKE] * 8), 0) == 1


def test_first_layer_geometries_take_the_first_layer_kernel(lib):
    """Every geometry of the first-layer parity tests resolves to the first-layer kernel,
    so those tests exercise it (and not a generic fallback)."""
    from test_gpu_parity import FIRST_LAYER_GEOMS
    L = cbr._load()
    L.cbr_plan_name.restype = ctypes.c_char_p
    for g in FIRST_LAYER_GEOMS:
        sp = cbr.make_shape(g.n, g.h, g.w, g.c, g.k, g.r, g.s, g.stride, g.pad, stride_w=g.stride_w, pad_w=g.pad_w)
        assert L.cbr_plan_name(L.cbr_plan_of(ctypes.byref(sp), 0)).decode() == "first_layer_c3s2", g


def test_plan_interface(lib):
    """Kernel plans: the defaults of the benchmark layers, eligibility, the override and its
    validation, and the compiled-in table's entries (each eligible for its shape)."""
    L = cbr._load()
    L.cbr_plan_name.restype = ctypes.c_char_p
    name = lambda p: L.cbr_plan_name(p).decode()
    head = cbr.make_shape(256, 56, 56, 64, 64, 3, 3, 1, 1)
    stem = cbr.make_shape(64, 224, 224, 3, 64, 7, 7, 2, 3)
    s4 = cbr.make_shape(256, 14, 14, 256, 256, 3, 3, 1, 1)
    assert name(L.cbr_plan_of(ctypes.byref(head), 0)) == "persistent_3x3_c64"
    assert name(L.cbr_plan_of(ctypes.byref(stem), 0)) == "first_layer_c3s2"
    assert name(L.cbr_plan_of(ctypes.byref(s4), 3)) == "wgrad_transposed_read"
    assert L.cbr_plan_eligible(ctypes.byref(head), 1, 1) == 0        # no statistics-free persistent form
    assert L.cbr_plan_eligible(ctypes.byref(head), 0, 7) == 0        # a weight-gradient plan on a conv stage
    assert L.cbr_plan_of(ctypes.byref(shp(k=12)), 0) == -3
    assert L.cbr_plan_of(ctypes.byref(head), 9) == -7
    assert L.cbr_set_plan_override(0, 99) == 7 and L.cbr_set_plan_override(5, 1) == 7
    try:
        assert L.cbr_set_plan_override(0, 6) == 0
        assert name(L.cbr_plan_of(ctypes.byref(head), 0)) == "generic_128x64"
        small = cbr.cbr_workspace_bytes(stem, cbr.CBR_OP_TRAIN)
        assert L.cbr_set_plan_override(0, 2) == 0                    # not eligible for s4: ignored there
        assert name(L.cbr_plan_of(ctypes.byref(s4), 0)) == "large_tile_224x256"
        assert small > 0
    finally:
        L.cbr_set_plan_override(0, 0)
    assert name(L.cbr_plan_of(ctypes.byref(head), 0)) == "persistent_3x3_c64"
    table = open(os.path.join(ROOT, "conv2d_batchnorm_relu_amd", "csrc", "cbr_tune_table.inc")).read()
    for row in re.findall(r"^\s*\{([-\d, ]+)\},", table, flags=re.M):
        st, n, h, w, c, k, r, s, sh, sw, ph, pw, plan = (int(v) for v in row.split(","))
        sp = cbr.make_shape(n, h, w, c, k, r, s, sh, ph, stride_w=sw, pad_w=pw)
        assert L.cbr_plan_eligible(ctypes.byref(sp), st, plan) == 1, row
        assert L.cbr_plan_of(ctypes.byref(sp), st) == plan, row


@pytest.mark.gpu
def test_binding_rejects_short_tensors():
    """A tensor with fewer elements than the call's shape implies (say, inputs drawn for a
    smaller batch) is refused by the binding before any kernel could run past its end."""
    import torch
    sp = cbr.make_shape(4, 8, 8, 64, 64, 3, 3, 1, 1)
    dev = "cuda"
    x_short = torch.zeros(2, 8, 8, 64, dtype=torch.bfloat16, device=dev)
    w = torch.zeros(64, 3, 3, 64, dtype=torch.bfloat16, device=dev)
    b = torch.zeros(64, device=dev)
    y = torch.empty(4, 8, 8, 64, dtype=torch.bfloat16, device=dev)
    with pytest.raises(cbr.CbrError, match="x holds 8192 elements, the shape needs 16384"):
        cbr.cbr_conv2d_bias_relu(sp, x_short, w, b, y)
    x = torch.zeros(4, 8, 8, 64, dtype=torch.bfloat16, device=dev)
    with pytest.raises(cbr.CbrError, match="y holds"):
        cbr.cbr_conv2d_bias(sp, x, w, b, y[:2])
    with pytest.raises(cbr.CbrError, match="bias holds"):
        cbr.cbr_conv2d_bias(sp, x, w, b[:32], y)


def test_draw_workload_geometry_matches_inputs():
    """A workload drawn at another batch size reports the geometry its inputs have."""
    from conv2d_batchnorm_relu_amd.inputs import draw_workload
    wl, d = draw_workload("s2_train", n=3)
    g = wl.geom
    assert g.n == 3 and d["x"].shape == (3, g.h, g.w, g.c) and d["w"].shape == (g.k, g.r, g.s, g.c)
    wl0, _ = draw_workload("tiny")
    assert wl0.geom.n == 2
