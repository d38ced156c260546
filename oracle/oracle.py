"""Python face of the fp64 CPU oracle (``convt3d_oracle.c``).  Test
infrastructure only: imported by tests, the smoke check and the benchmark's
CPU-baseline leg, never by the library path.

The C file is compiled with gcc/OpenMP into ``liboracle_convt3d.so`` next to
this file the first time it is needed (or by :func:`build`).  Arrays are numpy;
float32 inputs, float64 results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "convt3d_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_convt3d.so")
_lib = None

__all__ = [
    "build", "out_dim", "out_dims", "out_dim_general", "convt3d", "convt3d_general", "convt3d_gather",
    "convt3d_point",
    "relu_groupnorm", "softmax_sigmoid", "scale_bn_avgpool", "bn_running_update",
    "scale_bn_eval_avgpool", "run_workload",
    "num_threads", "OracleResult",
]


def build(force: bool = False) -> str:
    """Compile the oracle library with gcc -O2 -fopenmp (plain C, fp64)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        i, l, d = ctypes.c_int, ctypes.c_long, ctypes.c_double
        vp = ctypes.c_void_p
        lib.oracle_out_dim.restype = l
        lib.oracle_out_dim.argtypes = [l, l, l, l, l]
        conv_args = [vp, vp, vp, i, i, i, i, i, i, i, i, i, i, vp]
        lib.oracle_convt3d.restype = None
        lib.oracle_convt3d.argtypes = conv_args
        lib.oracle_convt3d_gather.restype = None
        lib.oracle_convt3d_gather.argtypes = conv_args
        lib.oracle_convt3d_point.restype = d
        lib.oracle_convt3d_point.argtypes = [vp, vp, vp] + [i] * 10 + [i, i, l, l, l]
        lib.oracle_out_dim_general.restype = l
        lib.oracle_out_dim_general.argtypes = [l, l, l, l, l, l]
        lib.oracle_convt3d_general.restype = None
        lib.oracle_convt3d_general.argtypes = [vp, vp, vp] + [i] * 6 + [vp] * 5 + [i, vp]
        lib.oracle_relu_groupnorm.restype = None
        lib.oracle_relu_groupnorm.argtypes = [vp, i, i, l, i, d, vp, vp, vp, vp]
        lib.oracle_softmax_sigmoid.restype = None
        lib.oracle_softmax_sigmoid.argtypes = [vp, i, i, l, vp, vp]
        lib.oracle_scale_bn_avgpool.restype = None
        lib.oracle_scale_bn_avgpool.argtypes = [vp, i, i, l, d, d, vp, vp, vp, vp]
        lib.oracle_bn_running_update.restype = None
        lib.oracle_bn_running_update.argtypes = [vp, i, d, d, vp, vp]
        lib.oracle_scale_bn_eval_avgpool.restype = None
        lib.oracle_scale_bn_eval_avgpool.argtypes = [vp, i, i, l, d, d, vp, vp, vp, vp, vp]
        lib.oracle_num_threads.restype = i
        lib.oracle_num_threads.argtypes = []
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def out_dim(n_in: int, k: int, s: int, p: int, op: int) -> int:
    return int(_load().oracle_out_dim(n_in, k, s, p, op))


def out_dims(d, h, w, k, s, p, op):
    return tuple(out_dim(v, k, s, p, op) for v in (d, h, w))


def _triple(v):
    return tuple(int(a) for a in v) if isinstance(v, (tuple, list)) else (int(v),) * 3


def out_dim_general(n_in: int, k: int, s: int, p: int, op: int, dl: int = 1) -> int:
    return int(_load().oracle_out_dim_general(n_in, k, s, p, op, dl))


def convt3d_general(x, w, b=None, stride=1, pad=0, out_pad=0, dilation=1, groups=1) -> np.ndarray:
    """Scatter-form transposed convolution for the general geometry: stride,
    pad, out_pad and dilation may be ints or (d, h, w) triples; w is
    [Cin, Cout/groups, kD, kH, kW].  fp64 result [N, Cout, Do, Ho, Wo]."""
    x, w, b = _f32(x), _f32(w), _f32(b)
    N, Cin, D, H, W = x.shape
    Cin2, Cog, kd, kh, kw = w.shape
    assert Cin == Cin2 and Cin % groups == 0
    Cout = Cog * groups
    k, s, p, op, dl = (kd, kh, kw), _triple(stride), _triple(pad), _triple(out_pad), _triple(dilation)
    od = tuple(out_dim_general(n, *a) for n, a in zip((D, H, W), zip(k, s, p, op, dl)))
    if min(od) <= 0:
        raise ValueError("empty transposed-convolution output")
    y = np.empty((N, Cout) + od, dtype=np.float64)
    arr = lambda t: (ctypes.c_int * 3)(*t)
    _load().oracle_convt3d_general(_ptr(x), _ptr(w), _ptr(b), N, Cin, Cout, D, H, W, arr(k), arr(s), arr(p),
                                   arr(op), arr(dl), groups, _ptr(y))
    return y


def _conv(fn, x, w, b, s, p, op):
    x, w, b = _f32(x), _f32(w), _f32(b)
    N, Cin, D, H, W = x.shape
    Cin2, Cout, k, k2, k3 = w.shape
    assert Cin == Cin2 and k == k2 == k3
    Do, Ho, Wo = out_dims(D, H, W, k, s, p, op)
    if min(Do, Ho, Wo) <= 0:
        raise ValueError("empty transposed-convolution output")
    y = np.empty((N, Cout, Do, Ho, Wo), dtype=np.float64)
    fn(_ptr(x), _ptr(w), _ptr(b), N, Cin, Cout, D, H, W, k, s, p, op, _ptr(y))
    return y


def convt3d(x, w, b=None, stride=1, pad=0, out_pad=0) -> np.ndarray:
    """Scatter-form transposed convolution, fp64 result [N, Cout, Do, Ho, Wo]."""
    return _conv(_load().oracle_convt3d, x, w, b, stride, pad, out_pad)


def convt3d_gather(x, w, b=None, stride=1, pad=0, out_pad=0) -> np.ndarray:
    """Gather-form transposed convolution (small inputs only)."""
    return _conv(_load().oracle_convt3d_gather, x, w, b, stride, pad, out_pad)


def convt3d_point(x, w, b, stride, pad, out_pad, n, co, od, oh, ow) -> float:
    """One output value by the gather form (x, w, b must be float32 C-contiguous)."""
    N, Cin, D, H, W = x.shape
    _, Cout, k, _, _ = w.shape
    assert x.dtype == np.float32 and w.dtype == np.float32 and x.flags.c_contiguous
    return float(_load().oracle_convt3d_point(_ptr(x), _ptr(w), _ptr(b), N, Cin, Cout, D, H, W,
                                              k, stride, pad, out_pad, n, co, od, oh, ow))


def relu_groupnorm(y, groups, eps=1e-5, gamma=None, beta=None):
    """ReLU then GroupNorm on fp64 y; returns (out, stats[N, G, 2] = mean, rstd)."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    N, C = y.shape[:2]
    S = int(np.prod(y.shape[2:]))
    assert C % groups == 0
    out = np.empty_like(y)
    stats = np.empty((N, groups, 2), dtype=np.float64)
    _load().oracle_relu_groupnorm(_ptr(y), N, C, S, groups, eps, _ptr(_f32(gamma)),
                                  _ptr(_f32(beta)), _ptr(out), _ptr(stats))
    return out, stats


def softmax_sigmoid(y):
    """Channel softmax then sigmoid on fp64 y; returns (out, softmax values)."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    N, C = y.shape[:2]
    S = int(np.prod(y.shape[2:]))
    out = np.empty_like(y)
    p = np.empty_like(y)
    _load().oracle_softmax_sigmoid(_ptr(y), N, C, S, _ptr(out), _ptr(p))
    return out, p


def scale_bn_avgpool(y, scale=1.0, eps=1e-5, gamma=None, beta=None):
    """x scale, training BatchNorm3d, global average pool; returns
    (out[N, C], stats[C, 2] = batch mean, biased variance of the scaled input)."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    N, C = y.shape[:2]
    S = int(np.prod(y.shape[2:]))
    out = np.empty((N, C), dtype=np.float64)
    stats = np.empty((C, 2), dtype=np.float64)
    _load().oracle_scale_bn_avgpool(_ptr(y), N, C, S, scale, eps, _ptr(_f32(gamma)),
                                    _ptr(_f32(beta)), _ptr(out), _ptr(stats))
    return out, stats


def bn_running_update(stats, count, momentum=0.1, rmean=None, rvar=None):
    """Running mean / variance after one training step from batch stats [C, 2]
    (mean, biased variance) over ``count`` values per channel; rmean/rvar
    default to a fresh module's 0 / 1.  Returns fp64 (rmean, rvar)."""
    stats = np.ascontiguousarray(stats, dtype=np.float64)
    C = stats.shape[0]
    rm = np.zeros(C) if rmean is None else np.array(rmean, dtype=np.float64)
    rv = np.ones(C) if rvar is None else np.array(rvar, dtype=np.float64)
    _load().oracle_bn_running_update(_ptr(stats), C, float(count), float(momentum), _ptr(rm), _ptr(rv))
    return rm, rv


def scale_bn_eval_avgpool(y, scale=1.0, eps=1e-5, gamma=None, beta=None, rmean=None, rvar=None):
    """x scale, BatchNorm3d with running statistics (eval mode), global average
    pool; returns out[N, C] (fp64)."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    N, C = y.shape[:2]
    S = int(np.prod(y.shape[2:]))
    out = np.empty((N, C), dtype=np.float64)
    _load().oracle_scale_bn_eval_avgpool(_ptr(y), N, C, S, scale, eps, _ptr(_f32(gamma)), _ptr(_f32(beta)),
                                         _ptr(_f32(rmean)), _ptr(_f32(rvar)), _ptr(out))
    return out


@dataclass
class OracleResult:
    y: np.ndarray                 # raw transposed-convolution output, fp64
    out: np.ndarray               # final output, fp64
    stats: Optional[np.ndarray]   # GN [N,G,2] (mean, rstd) | BN [C,2] (mean, var) | None
    p: Optional[np.ndarray] = None  # softmax values (softmax epilogue only)
    running: Optional[tuple] = None  # BN training: updated (running mean, running var), fp64


def run_workload(wl, inp) -> OracleResult:
    """The whole path for a workload description (epilogue codes as in
    ``activation_epilogues_amd.workloads``: 0 none, 1 ReLU+GroupNorm,
    2 softmax+sigmoid, 3 scale+BatchNorm(train)+avgpool, 4 scale+BatchNorm(eval,
    running statistics)+avgpool).  For code 3 with running statistics in the
    inputs, the result also carries them after the step's update."""
    if wl.is_cubic:
        y = convt3d(inp.x, inp.w, inp.b, wl.stride, wl.pad, wl.out_pad)
    else:
        y = convt3d_general(inp.x, inp.w, inp.b, wl.stride, wl.pad, wl.out_pad, wl.dilation, wl.conv_groups)
    if wl.epi == 0:
        return OracleResult(y, y, None)
    if wl.epi == 1:
        out, st = relu_groupnorm(y, wl.groups, wl.eps, inp.gamma, inp.beta)
        return OracleResult(y, out, st)
    if wl.epi == 2:
        out, p = softmax_sigmoid(y)
        return OracleResult(y, out, None, p)
    if wl.epi == 3:
        out, st = scale_bn_avgpool(y, wl.scale, wl.eps, inp.gamma, inp.beta)
        running = None
        if inp.rmean is not None:
            count = y.shape[0] * int(np.prod(y.shape[2:]))
            running = bn_running_update(st, count, wl.momentum, inp.rmean, inp.rvar)
        return OracleResult(y, out, st, running=running)
    if wl.epi == 4:
        out = scale_bn_eval_avgpool(y, wl.scale, wl.eps, inp.gamma, inp.beta, inp.rmean, inp.rvar)
        return OracleResult(y, out, None)
    raise ValueError(wl.epi)
