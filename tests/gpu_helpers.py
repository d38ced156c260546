"""Shared plumbing of the GPU tests: run the HIP path through the C ABI on
seeded inputs, run the oracle on the same inputs, compare."""
import sys

import numpy as np

from activation_epilogues_amd import convt3d as C
from activation_epilogues_amd import workloads as W

TOL = 1e-4  # max |err| of every fp32 output against the fp64 oracle


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def geom_of(wl):
    return C.make_geom(wl.n, wl.cin, wl.cout, wl.d, wl.h, wl.w, wl.k, wl.stride, wl.pad, wl.out_pad,
                       wl.dilation, wl.conv_groups)


def to_dev(a):
    import torch
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def run_gpu(wl, inp, kind=None, want_stats=True, stream=None):
    """One prepack + fused call through the C ABI; returns (out, stats) as numpy."""
    import torch
    kind = wl.epi if kind is None else kind
    g = geom_of(wl)
    call = C.FusedCall(g, kind, wl.groups, wl.eps, wl.scale, want_stats=want_stats)
    x, w, b = to_dev(inp.x), to_dev(inp.w), to_dev(inp.b)
    gamma, beta = to_dev(inp.gamma), to_dev(inp.beta)
    call.prepack(w, stream)
    # every output, exported statistic and workspace word starts as NaN: an
    # output the kernels leave unwritten, or a partial sum read without having
    # been written, shows up in the comparison
    call.out.fill_(float("nan"))
    call.workspace.fill_(float("nan"))
    if call.stats is not None:
        call.stats.fill_(float("nan"))
    torch.cuda.synchronize()
    out = call(x, b, gamma, beta, stream)
    torch.cuda.synchronize()
    st = None if call.stats is None else call.stats.cpu().numpy()
    return out.cpu().numpy(), st, call


def max_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    return float(np.abs(a - b).max()) if a.size else 0.0
