"""fp64 CPU oracle for the fused Conv2D -> BatchNorm -> ReLU operator.

TEST INFRASTRUCTURE ONLY: the test-suite, the package smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product (the HIP library under
``conv2d_batchnorm_relu_amd`` and its binding) never imports this package.

The arithmetic lives in ``cbr_oracle.c`` (plain C, fp64, OpenMP over the outermost
independent loops); this module only builds it and marshals numpy arrays.  Every
function here is the definition it names -- see the C file for the page passage each
one follows.  All arrays are float64 (masks uint8, one byte per element), layouts
NHWC for activations, KRSC for filters, NPQK for the conv output.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from collections import namedtuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cbr_oracle.c")
_LIB = os.path.join(_HERE, "libcbr_oracle.so")

# Problem geometry: input N,H,W,C; filter K,R,S (KRSC); stride and zero padding.
OShape = namedtuple("OShape", "n h w c k r s sh sw ph pw")


def out_hw(sp: OShape):
    """Output height/width: floor((in + 2*pad - k)/stride) + 1."""
    return (sp.h + 2 * sp.ph - sp.r) // sp.sh + 1, (sp.w + 2 * sp.pw - sp.s) // sp.sw + 1


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no fast-math: IEEE fp64 semantics kept)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None
_D = ctypes.POINTER(ctypes.c_double)
_U8 = ctypes.POINTER(ctypes.c_uint8)
_I64 = ctypes.POINTER(ctypes.c_int64)
_GEOM = [ctypes.c_int] * 11


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        lib.cbro_conv2d.argtypes = _GEOM + [_D, _D, _D, _D]
        lib.cbro_conv2d_at.argtypes = _GEOM + [_D, _D, _D, ctypes.c_long, _I64, _D]
        lib.cbro_conv2d_bias_act.argtypes = _GEOM + [_D, _D, _D, ctypes.c_int, _D]
        lib.cbro_batch_stats.argtypes = [ctypes.c_long, ctypes.c_int, _D, _D, _D]
        lib.cbro_forward_train.argtypes = _GEOM + [_D, _D, _D, _D, _D, _D, ctypes.c_double,
                                                   ctypes.c_double, _D, _D, _U8, _D, _D, _D, _D, _D]
        lib.cbro_forward_infer.argtypes = _GEOM + [_D, _D, _D, _D, _D, _D, _D, ctypes.c_double, _D, _D]
        lib.cbro_fold.argtypes = [ctypes.c_int] * 4 + [_D, _D, _D, _D, _D, _D, ctypes.c_double, _D, _D]
        lib.cbro_bn_backward.argtypes = [ctypes.c_long, ctypes.c_int, _D, _U8, _D, _D, _D, _D, _D, _D, _D]
        lib.cbro_conv2d_dgrad.argtypes = _GEOM + [_D, _D, _D]
        lib.cbro_conv2d_wgrad.argtypes = _GEOM + [_D, _D, _D]
        lib.cbro_backward.argtypes = _GEOM + [_D, _D, _D, _U8, _D, _D, _D, _D, _D, _D, _D, _D, _D]
        lib.cbro_num_threads.restype = ctypes.c_int
        lib.cbro_set_num_threads.argtypes = [ctypes.c_int]
        lib.cbro_set_num_threads.restype = None
        for f in ("cbro_conv2d", "cbro_conv2d_at", "cbro_batch_stats", "cbro_forward_train",
                  "cbro_forward_infer", "cbro_fold", "cbro_bn_backward", "cbro_conv2d_dgrad",
                  "cbro_conv2d_wgrad", "cbro_backward"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    if a is None:
        return None
    return a.ctypes.data_as(_D)


def _pu8(a):
    return a.ctypes.data_as(_U8)


def _g(sp: OShape):
    return tuple(int(v) for v in sp)


def num_threads() -> int:
    return _load().cbro_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of later oracle calls (timing only: results do not depend on it)."""
    _load().cbro_set_num_threads(int(n))


def conv2d(sp: OShape, x, w, bias=None):
    """z = conv(x, w) + bias; x NHWC, w KRSC -> z NPQK (fp64)."""
    x, w = _f64(x), _f64(w)
    b = None if bias is None else _f64(bias)
    P, Q = out_hw(sp)
    z = np.empty((sp.n, P, Q, sp.k), np.float64)
    _load().cbro_conv2d(*_g(sp), _p(x), _p(w), _p(b), _p(z))
    return z


def conv2d_bias_act(sp: OShape, x, w, bias=None, relu=True):
    """y = conv(x, w) + bias, then max(y, 0) when relu (fp64)."""
    x, w = _f64(x), _f64(w)
    b = None if bias is None else _f64(bias)
    P, Q = out_hw(sp)
    y = np.empty((sp.n, P, Q, sp.k), np.float64)
    _load().cbro_conv2d_bias_act(*_g(sp), _p(x), _p(w), _p(b), int(bool(relu)), _p(y))
    return y


def conv2d_at(sp: OShape, x, w, idx, bias=None):
    """conv(x, w) + bias evaluated only at the given linear NPQK indices."""
    x, w = _f64(x), _f64(w)
    b = None if bias is None else _f64(bias)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.shape[0], np.float64)
    _load().cbro_conv2d_at(*_g(sp), _p(x), _p(w), _p(b), idx.shape[0], idx.ctypes.data_as(_I64), _p(out))
    return out


def batch_stats(z2d):
    """Per-column mean and biased variance of an [M][K] array (two-pass, fp64)."""
    z2d = _f64(z2d)
    M, K = z2d.shape
    mean, var = np.empty(K), np.empty(K)
    _load().cbro_batch_stats(M, K, _p(z2d), _p(mean), _p(var))
    return mean, var


def forward_train(sp: OShape, x, w, gamma, beta, run_mean, run_var, eps, momentum):
    """Training forward; returns dict z, y, mask(uint8), mean, var, invstd, run_mean, run_var."""
    x, w, gamma, beta = _f64(x), _f64(w), _f64(gamma), _f64(beta)
    rm, rv = _f64(run_mean), _f64(run_var)
    P, Q = out_hw(sp)
    K = sp.k
    z = np.empty((sp.n, P, Q, K))
    y = np.empty_like(z)
    mask = np.empty(z.shape, np.uint8)
    var, mean, invstd, rmo, rvo = (np.empty(K) for _ in range(5))
    _load().cbro_forward_train(*_g(sp), _p(x), _p(w), _p(gamma), _p(beta), _p(rm), _p(rv),
                               float(eps), float(momentum), _p(z), _p(y), _pu8(mask), _p(var),
                               _p(mean), _p(invstd), _p(rmo), _p(rvo))
    return dict(z=z, y=y, mask=mask, mean=mean, var=var, invstd=invstd, run_mean=rmo, run_var=rvo)


def forward_infer(sp: OShape, x, w, bias, gamma, beta, run_mean, run_var, eps):
    """Inference forward by definition (running statistics, no fold)."""
    x, w = _f64(x), _f64(w)
    b = None if bias is None else _f64(bias)
    P, Q = out_hw(sp)
    zs = np.empty((sp.n, P, Q, sp.k))
    y = np.empty_like(zs)
    _load().cbro_forward_infer(*_g(sp), _p(x), _p(w), _p(b), _p(_f64(gamma)), _p(_f64(beta)),
                               _p(_f64(run_mean)), _p(_f64(run_var)), float(eps), _p(zs), _p(y))
    return y


def fold(w, bias, gamma, beta, run_mean, run_var, eps):
    """The BN fold: returns (w_fold KRSC, b_fold [K])."""
    w = _f64(w)
    K, R, S, C = w.shape
    b = None if bias is None else _f64(bias)
    wf = np.empty_like(w)
    bf = np.empty(K)
    _load().cbro_fold(K, R, S, C, _p(w), _p(b), _p(_f64(gamma)), _p(_f64(beta)),
                      _p(_f64(run_mean)), _p(_f64(run_var)), float(eps), _p(wf), _p(bf))
    return wf, bf


def bn_backward(dy, mask, z, gamma, saved_mean, saved_invstd):
    """ReLU-masked BN backward on [M][K] views; returns (dz, dgamma, dbeta)."""
    K = z.shape[-1]
    dy2, z2 = _f64(dy).reshape(-1, K), _f64(z).reshape(-1, K)
    m2 = np.ascontiguousarray(mask, dtype=np.uint8).reshape(-1, K)
    M = z2.shape[0]
    dz = np.empty_like(z2)
    dg, db = np.empty(K), np.empty(K)
    _load().cbro_bn_backward(M, K, _p(dy2), _pu8(m2), _p(z2), _p(_f64(gamma)), _p(_f64(saved_mean)),
                             _p(_f64(saved_invstd)), _p(dz), _p(dg), _p(db))
    return dz.reshape(z.shape), dg, db


def conv2d_dgrad(sp: OShape, dz, w):
    """dx = adjoint of conv in x (any stride)."""
    dx = np.empty((sp.n, sp.h, sp.w, sp.c))
    _load().cbro_conv2d_dgrad(*_g(sp), _p(_f64(dz)), _p(_f64(w)), _p(dx))
    return dx


def conv2d_wgrad(sp: OShape, dz, x):
    """dw[k,r,s,c] = sum over output pixels of dz * shifted x."""
    dw = np.empty((sp.k, sp.r, sp.s, sp.c))
    _load().cbro_conv2d_wgrad(*_g(sp), _p(_f64(dz)), _p(_f64(x)), _p(dw))
    return dw


def backward(sp: OShape, x, w, z, mask, dy, gamma, saved_mean, saved_invstd, want_dx=True):
    """Whole CBR backward; returns dict dz, dgamma, dbeta, dw, dx (dx None if not wanted)."""
    P, Q = out_hw(sp)
    K = sp.k
    x, w, z, dy = _f64(x), _f64(w), _f64(z), _f64(dy)
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    dz = np.empty((sp.n, P, Q, K))
    dg, db = np.empty(K), np.empty(K)
    dw = np.empty((sp.k, sp.r, sp.s, sp.c))
    dx = np.empty((sp.n, sp.h, sp.w, sp.c)) if want_dx else None
    _load().cbro_backward(*_g(sp), _p(x), _p(w), _p(z), _pu8(mask), _p(dy), _p(_f64(gamma)),
                          _p(_f64(saved_mean)), _p(_f64(saved_invstd)), _p(dz), _p(dg), _p(db),
                          _p(dw), _p(dx))
    return dict(dz=dz, dgamma=dg, dbeta=db, dw=dw, dx=dx)
