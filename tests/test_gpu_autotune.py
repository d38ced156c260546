"""convt3d_autotune: the plan chosen by timing is as correct as any other.

Each case tunes a geometry no other test uses (the tuned plan is kept for the
rest of the process), then checks the next convt3d_fused call against the fp64
oracle to the same tolerance as the default plans."""
import numpy as np
import pytest

import oracle
from activation_epilogues_amd import workloads as W

from gpu_helpers import TOL, geom_of, max_err, say, to_dev

pytestmark = pytest.mark.gpu

CASES = {"k3s1_gn": dict(n=1, d=29), "k3s2_softmax": dict(n=1, d=13), "k5s1_bnpool": dict(n=2, d=13),
         "k4s2_gn": dict(n=1, d=29)}


@pytest.mark.parametrize("name", list(CASES))
def test_autotuned_plan_matches_oracle(name, monkeypatch):
    import torch
    from activation_epilogues_amd import convt3d as C
    wl = W.BY_NAME[name].with_(**CASES[name])
    inp = W.make_inputs(wl)
    say(f"[case] autotune {name} n={wl.n} d={wl.d}")
    call = C.FusedCall(geom_of(wl), wl.epi, wl.groups, wl.eps, wl.scale, want_stats=True)
    x, w, b = to_dev(inp.x), to_dev(inp.w), to_dev(inp.b)
    gamma, beta = to_dev(inp.gamma), to_dev(inp.beta)
    call.prepack(w)
    assert call.plan_info()["tuned"] == 0
    res = call.autotune(x, b, gamma, beta)
    say(f"  tuned: {res}")
    # the workspace convt3d_workspace_size reports fits every candidate
    # 12 configurations, then up to 8 border segmentations of the fastest
    assert 1 <= res["candidates"] <= 12 + 8
    assert 0 <= res["chosen"] < res["candidates"]
    assert res["chosen_ms"] > 0 and res["chosen_ms"] <= res["model_choice_ms"]
    info = call.plan_info()
    assert info["tuned"] == 1
    # the reported plan string forces the tuned plan again (profiling without tuning)
    with monkeypatch.context() as m:
        m.setenv("CONVT3D_PLAN", C.plan_string(info))
        m.setenv("CONVT3D_PHASE_LOOP", str(info["phase_loop"]))
        forced = C.convt3d_get_plan_info(geom_of(wl), C.make_epilogue(wl.epi, wl.groups))
    assert {k: v for k, v in forced.items() if k != "tuned"} == {k: v for k, v in info.items() if k != "tuned"}
    call.out.fill_(float("nan"))
    out = call(x, b, gamma, beta)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ref = oracle.run_workload(wl, inp)
    assert max_err(out, ref.out.reshape(out.shape)) <= TOL
    if call.stats is not None:
        st = call.stats.cpu().numpy()
        np.testing.assert_allclose(st, ref.stats.reshape(st.shape), rtol=1e-5, atol=1e-6)
