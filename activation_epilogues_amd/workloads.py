"""Seeded synthetic workloads for the transposed-convolution + epilogue path.

This module is the only code shared by the oracle side and the HIP side: it
describes the five workload shapes and draws their inputs.  It holds none of
the method's arithmetic (no output-size formula, no convolution, no
normalisation); it only names shapes and draws random numbers.

Shapes follow the three problems the pages work on:
  * p61 page (ConvTranspose3d 64->128, k=3, then ReLU and GroupNorm(8)),
  * p49 page (ConvTranspose3d 32->64, k=3, stride 2, pad 1, output_padding 1,
    then softmax over channels and sigmoid),
  * p77 page (ConvTranspose3d 64->128, k=5, then x2.0, training-mode
    BatchNorm3d and AdaptiveAvgPool3d(1)),
plus a tiny GroupNorm case and a stride-2, k=4 GroupNorm case at 128 channels.

Input recipe (every workload): numpy ``default_rng(seed)`` draws, in this
order and as float64, x ~ N(0,1); w ~ U(-a, a) and b ~ U(-a, a) with
a = 1/sqrt(cin*k^3) (1/sqrt((cin/groups)*kD*kH*kW) in general); gamma ~ U(0.5, 1.5); beta ~ N(0, 0.1); then the
BatchNorm running statistics, running mean ~ N(0, 0.1) and running variance
~ U(0.5, 1.5) (the state of a module some steps into training; a fresh one
holds 0 and 1).  All seven arrays are always drawn (so the streams do not
depend on which are used) and then cast to float32.  The same float32 arrays
feed the oracle and the GPU.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

EPI_NONE = 0
EPI_RELU_GROUPNORM = 1
EPI_SOFTMAX_SIGMOID = 2
EPI_SCALE_BN_TRAIN_AVGPOOL = 3
EPI_SCALE_BN_EVAL_AVGPOOL = 4

EPI_NAMES = {
    EPI_NONE: "none",
    EPI_RELU_GROUPNORM: "relu_groupnorm",
    EPI_SOFTMAX_SIGMOID: "softmax_sigmoid",
    EPI_SCALE_BN_TRAIN_AVGPOOL: "scale_bn_train_avgpool",
    EPI_SCALE_BN_EVAL_AVGPOOL: "scale_bn_eval_avgpool",
}


def triple(v):
    """(d, h, w) values of an int or a 3-sequence."""
    return tuple(int(a) for a in v) if isinstance(v, (tuple, list)) else (int(v),) * 3


@dataclass(frozen=True)
class Workload:
    """One transposed-convolution + epilogue problem (NCDHW).  k, stride, pad,
    out_pad and dilation are ints (cubic) or (d, h, w) triples; conv_groups
    splits the channels as nn.ConvTranspose3d's `groups` does (groups is the
    GroupNorm group count)."""

    name: str
    n: int
    cin: int
    cout: int
    d: int
    h: int
    w: int
    k: object
    stride: object = 1
    pad: object = 0
    out_pad: object = 0
    bias: bool = True
    epi: int = EPI_RELU_GROUPNORM
    groups: int = 1
    eps: float = 1e-5
    scale: float = 1.0
    momentum: float = 0.1
    seed: int = 0
    dilation: object = 1
    conv_groups: int = 1
    note: str = field(default="", compare=False)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def kdims(self):
        return triple(self.k)

    @property
    def is_cubic(self) -> bool:
        """Cubic kernel, one stride / pad / out_pad for every dim, no dilation, one group."""
        return (all(len(set(triple(v))) == 1 for v in (self.k, self.stride, self.pad, self.out_pad))
                and triple(self.dilation) == (1, 1, 1) and self.conv_groups == 1)

    @property
    def x_shape(self):
        return (self.n, self.cin, self.d, self.h, self.w)

    @property
    def w_shape(self):
        return (self.cin, self.cout // self.conv_groups) + self.kdims


# The five workloads.  Seeds are 20260 + (position in this list, from 1).
WORKLOADS = [
    Workload("tiny_gn", 2, 8, 16, 8, 8, 8, k=3, stride=1, pad=0, bias=True,
             epi=EPI_RELU_GROUPNORM, groups=4, seed=20261,
             note="tiny GroupNorm case the oracle finishes in well under a second"),
    Workload("k3s1_gn", 16, 64, 128, 32, 32, 32, k=3, stride=1, pad=0, bias=False,
             epi=EPI_RELU_GROUPNORM, groups=8, seed=20262,
             note="p61 page shape: ConvTranspose3d 64->128 k3 (no bias), ReLU, GroupNorm(8)"),
    Workload("k3s2_softmax", 16, 32, 64, 16, 32, 32, k=3, stride=2, pad=1, out_pad=1,
             bias=True, epi=EPI_SOFTMAX_SIGMOID, seed=20263,
             note="p49 page shape: ConvTranspose3d 32->64 k3 s2 p1 op1, softmax(dim=1), sigmoid"),
    Workload("k5s1_bnpool", 16, 64, 128, 16, 32, 32, k=5, stride=1, pad=0, bias=True,
             epi=EPI_SCALE_BN_TRAIN_AVGPOOL, scale=2.0, seed=20264,
             note="p77 page shape: ConvTranspose3d 64->128 k5, x2, BatchNorm3d (train), avgpool"),
    Workload("k4s2_gn", 8, 128, 128, 32, 32, 32, k=4, stride=2, pad=1, bias=True,
             epi=EPI_RELU_GROUPNORM, groups=16, seed=20265,
             note="stride-2 k4 GroupNorm(16) case at 128 channels"),
]

# Further cases beyond the five, each on one of the pages' shapes: the p77
# layer with BatchNorm in evaluation mode (running statistics); the p61 layer
# with 4 channel groups and dilation 2 (nn.ConvTranspose3d's general form);
# the p49 layer with 256 output channels (more than one workgroup's softmax
# tile, so the softmax runs as a second pass).
EXTRA_WORKLOADS = [
    Workload("k5s1_bnpool_eval", 16, 64, 128, 16, 32, 32, k=5, stride=1, pad=0, bias=True,
             epi=EPI_SCALE_BN_EVAL_AVGPOOL, scale=2.0, seed=20264,
             note="p77 page shape with BatchNorm3d in eval mode (running statistics)"),
    Workload("k3s1_gn_g4_dl2", 16, 64, 128, 32, 32, 32, k=3, stride=1, pad=0, bias=False,
             epi=EPI_RELU_GROUPNORM, groups=8, seed=20266, dilation=2, conv_groups=4,
             note="p61 page shape with groups=4 and dilation=2"),
    Workload("k3s2_softmax_c256", 16, 32, 256, 16, 32, 32, k=3, stride=2, pad=1, out_pad=1, bias=True,
             epi=EPI_SOFTMAX_SIGMOID, seed=20267,
             note="p49 page shape with 256 output channels (softmax as a second pass)"),
]

BY_NAME = {wl.name: wl for wl in WORKLOADS + EXTRA_WORKLOADS}


@dataclass
class Inputs:
    x: np.ndarray
    w: np.ndarray
    b: Optional[np.ndarray]
    gamma: Optional[np.ndarray]
    beta: Optional[np.ndarray]
    rmean: Optional[np.ndarray] = None
    rvar: Optional[np.ndarray] = None


def make_inputs(wl: Workload, seed: Optional[int] = None, x_dist: str = "normal") -> Inputs:
    """Draw the float32 inputs of ``wl`` from ``default_rng(seed or wl.seed)``.

    ``x_dist`` may be "normal" (N(0,1), the default) or "uniform" (U[0,1)).
    Returned bias/gamma/beta are None when the workload does not use them.
    """
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    kd, kh, kw = wl.kdims
    a = 1.0 / np.sqrt(wl.cin // wl.conv_groups * kd * kh * kw)  # 1/sqrt(fan-in of one output)
    if x_dist == "normal":
        x = rng.standard_normal(wl.x_shape)
    elif x_dist == "uniform":
        x = rng.random(wl.x_shape)
    else:
        raise ValueError(x_dist)
    w = rng.uniform(-a, a, size=wl.w_shape)
    b = rng.uniform(-a, a, size=(wl.cout,))
    gamma = rng.uniform(0.5, 1.5, size=(wl.cout,))
    beta = rng.normal(0.0, 0.1, size=(wl.cout,))
    rmean = rng.normal(0.0, 0.1, size=(wl.cout,))
    rvar = rng.uniform(0.5, 1.5, size=(wl.cout,))
    f32 = lambda arr: np.ascontiguousarray(arr, dtype=np.float32)
    uses_affine = wl.epi in (EPI_RELU_GROUPNORM, EPI_SCALE_BN_TRAIN_AVGPOOL, EPI_SCALE_BN_EVAL_AVGPOOL)
    uses_running = wl.epi in (EPI_SCALE_BN_TRAIN_AVGPOOL, EPI_SCALE_BN_EVAL_AVGPOOL)
    return Inputs(
        x=f32(x),
        w=f32(w),
        b=f32(b) if wl.bias else None,
        gamma=f32(gamma) if uses_affine else None,
        beta=f32(beta) if uses_affine else None,
        rmean=f32(rmean) if uses_running else None,
        rvar=f32(rvar) if uses_running else None,
    )


def random_geometry(rng: np.random.Generator, max_in: int = 6, max_ch: int = 7,
                    epi: int = EPI_NONE) -> Workload:
    """A small random geometry for sweeps: k in 1..5, stride in 1..3,
    pad < k, out_pad < stride, odd sizes and channel counts that are not powers
    of two.  Some draws have an empty output; the caller decides (with its own
    size formula) whether to keep a draw."""
    k = int(rng.integers(1, 6))
    s = int(rng.integers(1, 4))
    p = int(rng.integers(0, k))
    op = int(rng.integers(0, s))
    d, h, w = (int(v) for v in rng.integers(1, max_in + 1, size=3))
    cin = int(rng.integers(1, max_ch + 1))
    cout = int(rng.integers(1, max_ch + 1))
    groups = 1
    if epi == EPI_RELU_GROUPNORM:
        divs = [g for g in range(1, cout + 1) if cout % g == 0]
        groups = int(rng.choice(divs))
    n = int(rng.integers(1, 4))
    return Workload("rand", n, cin, cout, d, h, w, k=k, stride=s, pad=p, out_pad=op,
                    bias=bool(rng.integers(0, 2)), epi=epi, groups=groups,
                    scale=float(rng.choice([1.0, 2.0, -0.5])),
                    seed=int(rng.integers(0, 2**31)))


def random_general_geometry(rng: np.random.Generator, max_in: int = 6, max_ch: int = 6,
                            epi: int = EPI_NONE) -> Workload:
    """A small random geometry with per-dim kernel sizes 1..4, strides 1..3,
    pads, output paddings (below max(stride, dilation)), dilations 1..3 and
    1..3 channel groups.  Some draws have an empty output; the caller decides
    (with its own size formula) whether to keep a draw."""
    k = tuple(int(v) for v in rng.integers(1, 5, size=3))
    s = tuple(int(v) for v in rng.integers(1, 4, size=3))
    dl = tuple(int(v) for v in rng.integers(1, 4, size=3))
    p = tuple(int(rng.integers(0, dl[i] * (k[i] - 1) + 1)) for i in range(3))
    op = tuple(int(rng.integers(0, max(s[i], dl[i]))) for i in range(3))
    d, h, w = (int(v) for v in rng.integers(1, max_in + 1, size=3))
    G = int(rng.integers(1, 4))
    cin = G * int(rng.integers(1, max_ch + 1))
    cout = G * int(rng.integers(1, max_ch + 1))
    groups = 1
    if epi == EPI_RELU_GROUPNORM:
        divs = [g for g in range(1, cout + 1) if cout % g == 0]
        groups = int(rng.choice(divs))
    n = int(rng.integers(1, 4))
    return Workload("rgen", n, cin, cout, d, h, w, k=k, stride=s, pad=p, out_pad=op, bias=bool(rng.integers(0, 2)),
                    epi=epi, groups=groups, scale=float(rng.choice([1.0, 2.0, -0.5])),
                    seed=int(rng.integers(0, 2**31)), dilation=dl, conv_groups=G)
