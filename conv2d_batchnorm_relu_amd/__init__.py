"""Fused Conv2D -> BatchNorm -> ReLU (CBR) for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libcbr.so`` (the HIP kernels and the C ABI declared in
``include/cbr.h``).  The functions carry the C names and only marshal arguments: torch
tensors are passed by device pointer, the stream defaults to torch's current stream.
All computation runs in the library's kernels; there is no CPU path, and every call
raises if the library has not been built.

Tensor conventions (see include/cbr.h): NHWC activations and KRSC filters as
``torch.bfloat16`` (or 16-bit integer tensors holding bf16 bits), float32 per-channel
vectors, an int32/uint32 packed ReLU mask of ``cbr_mask_words(shape)`` words, and a
caller-allocated device workspace of ``cbr_workspace_bytes(shape, op)`` bytes.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["CbrError", "CbrShape", "make_shape", "cbr_status_str", "cbr_output_hw", "cbr_mask_words",
           "cbr_workspace_bytes", "cbr_forward_train", "cbr_forward_infer", "cbr_backward",
           "cbr_conv2d_bias_relu", "cbr_conv2d_bias", "cbr_forward_train_noalloc",
           "CBR_OP_TRAIN", "CBR_OP_INFER", "CBR_OP_BWD", "library_path"]

CBR_OP_TRAIN, CBR_OP_INFER, CBR_OP_BWD = 0, 1, 2
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libcbr.so")


class CbrShape(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in
                ("n", "h", "w", "c", "k", "r", "s", "stride_h", "stride_w", "pad_h", "pad_w")]


class CbrError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str | None = None):
        self.status = status
        msg = detail if detail is not None else cbr_status_str(status)
        super().__init__(f"{where}: {msg} (status {status})")


_lib = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(the CBR operator has no CPU fallback)")
    # The library must resolve its HIP runtime to the one that owns the callers' device
    # memory and streams.  torch loads its own copy of the runtime; loading torch first
    # makes the library bind to that copy (same soname) instead of a second one.
    import torch  # noqa: F401
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    S = ctypes.POINTER(CbrShape)
    lib.cbr_status_str.argtypes = [ctypes.c_int]
    lib.cbr_status_str.restype = ctypes.c_char_p
    lib.cbr_output_hw.argtypes = [S, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.cbr_output_hw.restype = ctypes.c_int
    lib.cbr_mask_words.argtypes = [S]
    lib.cbr_mask_words.restype = ctypes.c_size_t
    lib.cbr_workspace_bytes.argtypes = [S, ctypes.c_int]
    lib.cbr_workspace_bytes.restype = ctypes.c_size_t
    lib.cbr_forward_train.argtypes = [S, P, P, P, P, P, P, ctypes.c_float, ctypes.c_float,
                                      P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.cbr_forward_train.restype = ctypes.c_int
    lib.cbr_forward_infer.argtypes = [S, P, P, P, P, P, P, P, ctypes.c_float, P, P, ctypes.c_size_t, P]
    lib.cbr_forward_infer.restype = ctypes.c_int
    lib.cbr_backward.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.cbr_backward.restype = ctypes.c_int
    lib.cbr_forward_train_ev.argtypes = lib.cbr_forward_train.argtypes + [P]
    lib.cbr_forward_train_ev.restype = ctypes.c_int
    lib.cbr_forward_infer_ev.argtypes = lib.cbr_forward_infer.argtypes + [P]
    lib.cbr_forward_infer_ev.restype = ctypes.c_int
    lib.cbr_backward_ev.argtypes = lib.cbr_backward.argtypes + [P]
    lib.cbr_backward_ev.restype = ctypes.c_int
    lib.cbr_forward_train_noalloc.argtypes = [S, P, P, P, P, P, P, ctypes.c_float, ctypes.c_float,
                                              P, P, P, P, P, P, P, P]
    lib.cbr_forward_train_noalloc.restype = ctypes.c_int
    for name in ("cbr_conv2d_bias_relu", "cbr_conv2d_bias"):
        fn, fe = getattr(lib, name), getattr(lib, name + "_ev")
        fn.argtypes = [S, P, P, P, P, P]
        fn.restype = ctypes.c_int
        fe.argtypes = fn.argtypes + [P]
        fe.restype = ctypes.c_int
    _lib = lib
    return lib


def make_shape(n, h, w, c, k, r, s, stride=1, pad=0, stride_w=None, pad_w=None) -> CbrShape:
    return CbrShape(n, h, w, c, k, r, s, stride, stride if stride_w is None else stride_w,
                    pad, pad if pad_w is None else pad_w)


def _sp(shape):
    return ctypes.byref(shape)


_E_VALUE = 7   # CBR_E_VALUE: the binding reports unusable tensors with it


def _ptr(t, itemsize, name, where, numel=None):
    """Device address of tensor t, after checking that the library can read it as the
    dense array of itemsize-byte elements that include/cbr.h describes: a CUDA (HIP)
    tensor, contiguous in its own layout, with that element size and at least numel
    elements (the count the call's shape implies, when known).  An integer is taken as a
    raw device address; None stays NULL."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise CbrError(_E_VALUE, where, f"{name} is not a GPU tensor")
    if not t.is_contiguous():
        raise CbrError(_E_VALUE, where, f"{name} is not contiguous (the library reads dense NHWC/KRSC arrays)")
    if t.element_size() != itemsize:
        raise CbrError(_E_VALUE, where, f"{name} has {t.element_size()}-byte elements, expected {itemsize}")
    if numel is not None and t.numel() < numel:
        raise CbrError(_E_VALUE, where, f"{name} holds {t.numel()} elements, the shape needs {numel}")
    return t.data_ptr()


def _extents(shape):
    """Element counts of a call's arrays for shape: x (NHWC), w (KRSC), out (NPQK: z, y,
    dy, dz), k (per-channel vectors), mask (32-bit words).  All None when the library
    rejects the shape: it then reports the shape's own error."""
    p, q = ctypes.c_int32(), ctypes.c_int32()
    if _load().cbr_output_hw(_sp(shape), ctypes.byref(p), ctypes.byref(q)) != 0:
        return dict.fromkeys(("x", "w", "out", "k", "mask"))
    s = shape
    return dict(x=s.n * s.h * s.w * s.c, w=s.k * s.r * s.s * s.c, out=s.n * p.value * q.value * s.k, k=s.k,
                mask=cbr_mask_words(shape))


def _ws(workspace, where):
    if workspace is None:
        return None, 0
    if isinstance(workspace, tuple):
        return workspace
    p = _ptr(workspace, workspace.element_size(), "workspace", where)
    return p, workspace.numel() * workspace.element_size()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, where):
    if status != 0:
        raise CbrError(status, where)


def cbr_status_str(status: int) -> str:
    return _load().cbr_status_str(int(status)).decode()


def cbr_output_hw(shape: CbrShape):
    p, q = ctypes.c_int32(), ctypes.c_int32()
    _check(_load().cbr_output_hw(_sp(shape), ctypes.byref(p), ctypes.byref(q)), "cbr_output_hw")
    return p.value, q.value


def cbr_mask_words(shape: CbrShape) -> int:
    return int(_load().cbr_mask_words(_sp(shape)))


def cbr_workspace_bytes(shape: CbrShape, op: int) -> int:
    return int(_load().cbr_workspace_bytes(_sp(shape), int(op)))


def _events(events):
    """A ctypes array of hipEvent_t handles (torch.cuda.Event objects or raw ints)."""
    if events is None:
        return None
    handles = [e if isinstance(e, int) else e.cuda_event for e in events]
    return (ctypes.c_void_p * len(handles))(*handles)


def cbr_forward_train(shape, x, w, gamma, beta, run_mean_in, run_var_in, eps, momentum,
                      z, y, relu_mask, saved_mean, saved_invstd, run_mean_out, run_var_out,
                      workspace, stream=None, events=None):
    f = "cbr_forward_train"
    ws, nbytes = _ws(workspace, f)
    e = _extents(shape)
    args = (_sp(shape), _ptr(x, 2, "x", f, e["x"]), _ptr(w, 2, "w", f, e["w"]), _ptr(gamma, 4, "gamma", f, e["k"]),
            _ptr(beta, 4, "beta", f, e["k"]), _ptr(run_mean_in, 4, "run_mean_in", f, e["k"]),
            _ptr(run_var_in, 4, "run_var_in", f, e["k"]), float(eps), float(momentum), _ptr(z, 2, "z", f, e["out"]),
            _ptr(y, 2, "y", f, e["out"]), _ptr(relu_mask, 4, "relu_mask", f, e["mask"]),
            _ptr(saved_mean, 4, "saved_mean", f, e["k"]), _ptr(saved_invstd, 4, "saved_invstd", f, e["k"]),
            _ptr(run_mean_out, 4, "run_mean_out", f, e["k"]), _ptr(run_var_out, 4, "run_var_out", f, e["k"]),
            ws, nbytes, _stream(stream))
    if events is None:
        _check(_load().cbr_forward_train(*args), f)
    else:
        _check(_load().cbr_forward_train_ev(*args, _events(events)), "cbr_forward_train_ev")


def cbr_forward_train_noalloc(shape, x, w, gamma, beta, run_mean_in, run_var_in, eps, momentum,
                              z, y, relu_mask, saved_mean, saved_invstd, run_mean_out, run_var_out, stream=None):
    f = "cbr_forward_train_noalloc"
    e = _extents(shape)
    args = (_sp(shape), _ptr(x, 2, "x", f, e["x"]), _ptr(w, 2, "w", f, e["w"]), _ptr(gamma, 4, "gamma", f, e["k"]),
            _ptr(beta, 4, "beta", f, e["k"]), _ptr(run_mean_in, 4, "run_mean_in", f, e["k"]),
            _ptr(run_var_in, 4, "run_var_in", f, e["k"]), float(eps), float(momentum), _ptr(z, 2, "z", f, e["out"]),
            _ptr(y, 2, "y", f, e["out"]), _ptr(relu_mask, 4, "relu_mask", f, e["mask"]),
            _ptr(saved_mean, 4, "saved_mean", f, e["k"]), _ptr(saved_invstd, 4, "saved_invstd", f, e["k"]),
            _ptr(run_mean_out, 4, "run_mean_out", f, e["k"]), _ptr(run_var_out, 4, "run_var_out", f, e["k"]),
            _stream(stream))
    _check(_load().cbr_forward_train_noalloc(*args), f)


def cbr_forward_infer(shape, x, w, conv_bias, gamma, beta, run_mean, run_var, eps, y,
                      workspace, stream=None, events=None):
    f = "cbr_forward_infer"
    ws, nbytes = _ws(workspace, f)
    e = _extents(shape)
    args = (_sp(shape), _ptr(x, 2, "x", f, e["x"]), _ptr(w, 2, "w", f, e["w"]),
            _ptr(conv_bias, 4, "conv_bias", f, e["k"]), _ptr(gamma, 4, "gamma", f, e["k"]),
            _ptr(beta, 4, "beta", f, e["k"]), _ptr(run_mean, 4, "run_mean", f, e["k"]),
            _ptr(run_var, 4, "run_var", f, e["k"]), float(eps), _ptr(y, 2, "y", f, e["out"]), ws, nbytes,
            _stream(stream))
    if events is None:
        _check(_load().cbr_forward_infer(*args), f)
    else:
        _check(_load().cbr_forward_infer_ev(*args, _events(events)), "cbr_forward_infer_ev")


def cbr_backward(shape, x, w, z, relu_mask, dy, gamma, saved_mean, saved_invstd,
                 dz, dgamma, dbeta, dw, dx, workspace, stream=None, events=None):
    f = "cbr_backward"
    ws, nbytes = _ws(workspace, f)
    e = _extents(shape)
    args = (_sp(shape), _ptr(x, 2, "x", f, e["x"]), _ptr(w, 2, "w", f, e["w"]), _ptr(z, 2, "z", f, e["out"]),
            _ptr(relu_mask, 4, "relu_mask", f, e["mask"]), _ptr(dy, 2, "dy", f, e["out"]),
            _ptr(gamma, 4, "gamma", f, e["k"]), _ptr(saved_mean, 4, "saved_mean", f, e["k"]),
            _ptr(saved_invstd, 4, "saved_invstd", f, e["k"]), _ptr(dz, 2, "dz", f, e["out"]),
            _ptr(dgamma, 4, "dgamma", f, e["k"]), _ptr(dbeta, 4, "dbeta", f, e["k"]), _ptr(dw, 4, "dw", f, e["w"]),
            _ptr(dx, 2, "dx", f, e["x"]), ws, nbytes, _stream(stream))
    if events is None:
        _check(_load().cbr_backward(*args), f)
    else:
        _check(_load().cbr_backward_ev(*args, _events(events)), "cbr_backward_ev")


def _conv_bias(name, shape, x, w, bias, y, stream, events):
    e = _extents(shape)
    args = (_sp(shape), _ptr(x, 2, "x", name, e["x"]), _ptr(w, 2, "w", name, e["w"]),
            _ptr(bias, 4, "bias", name, e["k"]), _ptr(y, 2, "y", name, e["out"]), _stream(stream))
    if events is None:
        _check(getattr(_load(), name)(*args), name)
    else:
        _check(getattr(_load(), name + "_ev")(*args, _events(events)), name + "_ev")


def cbr_conv2d_bias_relu(shape, x, w, bias, y, stream=None, events=None):
    _conv_bias("cbr_conv2d_bias_relu", shape, x, w, bias, y, stream, events)


def cbr_conv2d_bias(shape, x, w, bias, y, stream=None, events=None):
    _conv_bias("cbr_conv2d_bias", shape, x, w, bias, y, stream, events)
