"""Kernel timing sessions on the GPU: recording every kind or only some kinds
leaves the results bitwise unchanged, and only the requested kinds get
durations."""
import numpy as np
import pytest

from activation_epilogues_amd import workloads as W

from gpu_helpers import geom_of, say, to_dev

pytestmark = pytest.mark.gpu

KINDS = ("conv_ms", "finalize_ms", "normalize_ms", "reduce_ms", "prepack_ms")


def test_profile_kinds_record_only_the_requested_kernels():
    import torch
    from activation_epilogues_amd import convt3d as C
    wl = W.BY_NAME["tiny_gn"]
    inp = W.make_inputs(wl)
    say(f"[case] profile kinds {wl.name}")
    call = C.FusedCall(geom_of(wl), wl.epi, wl.groups, wl.eps, wl.scale)
    x, w, b = to_dev(inp.x), to_dev(inp.w), to_dev(inp.b)
    gamma, beta = to_dev(inp.gamma), to_dev(inp.beta)

    def step():
        call.prepack(w)
        out = call(x, b, gamma, beta)
        torch.cuda.synchronize()
        return out.cpu().numpy().copy()

    plain = step()
    results = {}
    for name, mask in (("all", C.PROFILE_ALL), ("conv", C.PROFILE_CONV),
                       ("finalize+normalize", C.PROFILE_FINALIZE | C.PROFILE_NORMALIZE)):
        if mask == C.PROFILE_ALL:
            C.convt3d_profile_begin()
        else:
            C.convt3d_profile_begin_kinds(mask)
        out = step()
        out = step()
        results[name] = C.convt3d_profile_end()
        assert np.array_equal(out, plain), name
    say(f"  {results}")
    r = results["all"]
    assert r["calls"] == 2
    assert r["conv_ms"] > 0 and r["finalize_ms"] > 0 and r["normalize_ms"] > 0 and r["prepack_ms"] > 0
    assert r["reduce_ms"] == 0
    r = results["conv"]
    assert r["calls"] == 2 and r["conv_ms"] > 0
    assert all(r[k] == 0 for k in KINDS if k != "conv_ms")
    r = results["finalize+normalize"]
    assert r["finalize_ms"] > 0 and r["normalize_ms"] > 0
    assert r["conv_ms"] == 0 and r["prepack_ms"] == 0 and r["reduce_ms"] == 0
