"""The allocation-free training forward (cbr_forward_train_noalloc) against the
workspace entry point (cbr_forward_train), through the C ABI: the same kernels run on
a library-held scratch array, so every output must be bit-identical.  Two calls in a
row, the second on a smaller input, so the second reads an array the first has filled."""
import ctypes

import numpy as np
import pytest
import torch

from conv2d_batchnorm_relu_amd.inputs import Geometry, draw
import cbr_harness as H

pytestmark = pytest.mark.gpu


def run_noalloc(g, d):
    import conv2d_batchnorm_relu_amd as cbr
    sp = H.cshape(g)
    x, w = H.dev_bf16(d["x"]), H.dev_bf16(d["w"])
    gamma, beta = H.dev_f32(d["gamma"]), H.dev_f32(d["beta"])
    rm_in, rv_in = H.dev_f32(d["run_mean"]), H.dev_f32(d["run_var"])
    z = H.empty_bf16((g.n, g.p, g.q, g.k))
    y = H.empty_bf16((g.n, g.p, g.q, g.k))
    mask = torch.full((cbr.cbr_mask_words(sp),), -1, dtype=torch.int32, device="cuda")
    sm, si, rmo, rvo = (H.empty_f32(g.k) for _ in range(4))
    st = cbr._load().cbr_forward_train_noalloc(
        ctypes.byref(sp), x.data_ptr(), w.data_ptr(), gamma.data_ptr(), beta.data_ptr(), rm_in.data_ptr(),
        rv_in.data_ptr(), 1e-5, 0.1, z.data_ptr(), y.data_ptr(), mask.data_ptr(), sm.data_ptr(), si.data_ptr(),
        rmo.data_ptr(), rvo.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, cbr.cbr_status_str(st)
    torch.cuda.synchronize()
    return dict(z=H.host_bf16(z), y=H.host_bf16(y), mask_words=mask.cpu().numpy().view(np.uint32),
                mean=sm.cpu().numpy(), invstd=si.cpu().numpy(), run_mean=rmo.cpu().numpy(),
                run_var=rvo.cpu().numpy())


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_noalloc_matches_workspace_entry_point():
    # persistent 3x3 conv (256 statistics rows), then a smaller generic-conv shape
    for g in (Geometry(300, 12, 16, 64, 64, 3, 3, 1, 1), Geometry(3, 9, 11, 16, 24, 3, 3, 1, 1)):
        H.log(f"no-alloc train forward {g}")
        d = draw(g, "train", 31)
        ref, _ = H.gpu_train(g, d)
        got = run_noalloc(g, d)
        for k in ("z", "y", "mask_words", "mean", "invstd", "run_mean", "run_var"):
            np.testing.assert_array_equal(got[k], ref[k], err_msg=f"{g}: {k}")
        H.check_train(g, d, got | {"mask": H.unpack_mask(torch.from_numpy(got["mask_words"].view(np.int32)),
                                                           g.m * g.k).reshape(g.n, g.p, g.q, g.k)},
                      H.oracle_train(g, d))

