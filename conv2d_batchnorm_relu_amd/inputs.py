"""Seeded synthetic inputs for the CBR operator (shared by tests and the benchmark).

This module holds no arithmetic of the operator itself: it only draws random tensors
(numpy PCG64, ``numpy.random.default_rng(seed)``) with the shapes and distributions of
the workloads, and rounds them to bfloat16 (round-to-nearest-even) so that the GPU and
the CPU oracle read exactly the same values.

Draw order for every workload: x, w, [conv bias], gamma, beta, [running stats], dy.

Workloads (NHWC activations, KRSC filters; ResNet-50 / VGG16BN-style conv layers at
ImageNet resolution stand in for real feature maps -- no dataset is used):
  tiny      N2  8x8   C4   -> K8   3x3 s1 p1  (fp32 draws; train fwd + bwd)
  stem      N64 224x224 C3 -> K64  7x7 s2 p3  (first layer, train fwd)
  s2_train  N256 56x56 C64 -> K64  3x3 s1 p1  (train fwd; the headline workload)
  s3_infer  N256 28x28 C128 -> K128 3x3 s1 p1 (folded-BN inference, conv bias)
  s4_bwd    N256 14x14 C256 -> K256 3x3 s1 p1 (train bwd after a train fwd)
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Geometry:
    n: int
    h: int
    w: int
    c: int
    k: int
    r: int
    s: int
    stride: int = 1               # vertical stride (both axes unless stride_w is given)
    pad: int = 1                  # vertical zero padding (both axes unless pad_w is given)
    stride_w: int | None = None   # horizontal stride when it differs from the vertical one
    pad_w: int | None = None      # horizontal padding when it differs from the vertical one

    @property
    def sh(self) -> int:
        return self.stride

    @property
    def sw(self) -> int:
        return self.stride if self.stride_w is None else self.stride_w

    @property
    def ph(self) -> int:
        return self.pad

    @property
    def pw(self) -> int:
        return self.pad if self.pad_w is None else self.pad_w

    @property
    def p(self) -> int:
        return (self.h + 2 * self.ph - self.r) // self.sh + 1

    @property
    def q(self) -> int:
        return (self.w + 2 * self.pw - self.s) // self.sw + 1

    @property
    def m(self) -> int:
        """Output pixels N*P*Q (GEMM rows, BN reduction length)."""
        return self.n * self.p * self.q

    def with_n(self, n: int) -> "Geometry":
        return replace(self, n=n)


@dataclass(frozen=True)
class Workload:
    name: str
    geom: Geometry
    call: str            # "train", "infer" or "bwd"
    seed: int
    bf16: bool = True
    eps: float = 1e-5
    momentum: float = 0.1


WORKLOADS = {
    "tiny": Workload("tiny", Geometry(2, 8, 8, 4, 8, 3, 3, 1, 1), "train", 1, bf16=False),
    "stem": Workload("stem", Geometry(64, 224, 224, 3, 64, 7, 7, 2, 3), "train", 2),
    "s2_train": Workload("s2_train", Geometry(256, 56, 56, 64, 64, 3, 3, 1, 1), "train", 3),
    "s3_infer": Workload("s3_infer", Geometry(256, 28, 28, 128, 128, 3, 3, 1, 1), "infer", 4),
    "s4_bwd": Workload("s4_bwd", Geometry(256, 14, 14, 256, 256, 3, 3, 1, 1), "bwd", 5),
}


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # finite inputs: u + 0x8000 cannot wrap past 2^32
    r = (u >> 16) & np.uint32(1)
    r += u
    r += np.uint32(0x7FFF)
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bfloat16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(bits).astype(np.uint32) << 16).view(np.float32)


def draw(geom: Geometry, call: str, seed: int, bf16: bool = True) -> dict:
    """Draw one seeded input set.  Values are float32 arrays; with bf16=True they are
    exactly bfloat16-representable (x, w, dy rounded; gamma/beta/stats stay float32).

    x ~ N(0,1) NHWC; w ~ U(-a, a), a = sqrt(6 / (C*R*S)) (Kaiming-uniform, ReLU gain)
    KRSC; conv bias ~ U(-0.1, 0.1) for inference, absent otherwise; gamma ~ U(0.5, 1.5);
    beta ~ U(-0.5, 0.5); running stats: mean 0 / var 1 for training, mean ~ N(0, 0.5)
    (standard deviation 0.5) and var ~ U(0.5, 2) for inference; dy ~ N(0,1) for the
    backward call.
    """
    g = geom
    rng = np.random.default_rng(seed)
    out = {}
    x = rng.standard_normal((g.n, g.h, g.w, g.c), dtype=np.float32)
    a = np.sqrt(6.0 / (g.c * g.r * g.s))
    w = rng.uniform(-a, a, size=(g.k, g.r, g.s, g.c)).astype(np.float32)
    out["x"] = bf16_round(x) if bf16 else x
    out["w"] = bf16_round(w) if bf16 else w
    if call == "infer":
        out["bias"] = rng.uniform(-0.1, 0.1, size=g.k).astype(np.float32)
    out["gamma"] = rng.uniform(0.5, 1.5, size=g.k).astype(np.float32)
    out["beta"] = rng.uniform(-0.5, 0.5, size=g.k).astype(np.float32)
    if call == "infer":
        out["run_mean"] = rng.normal(0.0, 0.5, size=g.k).astype(np.float32)
        out["run_var"] = rng.uniform(0.5, 2.0, size=g.k).astype(np.float32)
    else:
        out["run_mean"] = np.zeros(g.k, np.float32)
        out["run_var"] = np.ones(g.k, np.float32)
    if call == "bwd" or (call == "train" and not bf16):
        dy = rng.standard_normal((g.n, g.p, g.q, g.k), dtype=np.float32)
        out["dy"] = bf16_round(dy) if bf16 else dy
    return out


def draw_workload(name: str, n: int | None = None) -> tuple[Workload, dict]:
    """Inputs of a named workload, optionally with another batch size (same recipe).  The
    returned workload's geometry is the one the inputs were drawn for."""
    wl = WORKLOADS[name]
    if n is not None:
        wl = replace(wl, geom=wl.geom.with_n(n))
    return wl, draw(wl.geom, wl.call, wl.seed, wl.bf16)
