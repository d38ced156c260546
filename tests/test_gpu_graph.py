"""The library under HIP graph capture: convt3d_prepack_weights +
convt3d_fused enqueue kernels only (no allocation, no memset, no host wait), so
a caller can capture a step and replay it.  Each replay is compared bitwise
with the eager result (the kernels are deterministic), with eager work and
synchronisations between replays."""
import numpy as np
import pytest

from activation_epilogues_amd import convt3d as C
from activation_epilogues_amd import workloads as W

from gpu_helpers import geom_of, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", [W.EPI_RELU_GROUPNORM, W.EPI_SOFTMAX_SIGMOID, W.EPI_SCALE_BN_TRAIN_AVGPOOL,
                                  W.EPI_SCALE_BN_EVAL_AVGPOOL])
def test_fused_step_replays_from_a_graph(kind):
    import torch
    wl = W.Workload("graph", 2, 12, 40, 6, 7, 8, k=3, stride=2, pad=1, out_pad=1, bias=True, epi=kind,
                    groups=4 if kind == W.EPI_RELU_GROUPNORM else 1, scale=2.0, seed=9300 + kind)
    say(f"[case] graph capture kind {kind}")
    inp = W.make_inputs(wl)
    call = C.FusedCall(geom_of(wl), wl.epi, wl.groups, wl.eps, wl.scale, want_stats=True)
    x, w, b = to_dev(inp.x), to_dev(inp.w), to_dev(inp.b)
    gamma, beta = to_dev(inp.gamma), to_dev(inp.beta)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        # eager reference (also sets each kernel's LDS attribute before capture)
        call.prepack(w, stream)
        call(x, b, gamma, beta, stream)
        stream.synchronize()
        want = call.out.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            call.prepack(w, stream)
            call(x, b, gamma, beta, stream)
    torch.cuda.synchronize()
    for rep in range(3):
        call.out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(call.out, want), f"replay {rep} differs"
        _ = (x * 2.0).sum().item()  # unrelated eager work between replays
