"""GPU parity at the full workload sizes: with the cost model's first plan
(what convt3d_fused runs before any tuning) and with the plan convt3d_autotune
picks on the full-size buffers (the launch configuration the benchmark times,
since bench.py tunes before its warm-up).  Expected values were written by
tests/golden/make_full_size_golden.py, which runs only the fp64 oracle:
sampled voxels of the raw convolution and of the final output, the exported
statistics, and for the pooled BatchNorm path the whole [n, cout] output.
Properties that hold at any size are checked on the whole GPU output."""
import os

import numpy as np
import pytest

from activation_epilogues_amd import workloads as W

from gpu_helpers import TOL, max_err, run_gpu, say

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
# the four conv workloads, then the two general-geometry ones (the p61 layer
# with 4 groups and dilation 2; the p49 layer with 256 channels)
NAMES = ["k3s1_gn", "k3s2_softmax", "k5s1_bnpool", "k4s2_gn", "k3s1_gn_g4_dl2", "k3s2_softmax_c256"]


def load_golden(name):
    path = os.path.join(GOLDEN, f"full_{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    return np.load(path, allow_pickle=False)


def check_inputs(g, inp):
    for k in ("x", "w", "b", "gamma", "beta"):
        a = getattr(inp, k)
        if "sum_" + k in g.files:
            assert a is not None
            assert np.array_equal(a.reshape(-1)[:8], g["head_" + k]), k
            assert a.astype(np.float64).sum() == g["sum_" + k], k


@pytest.mark.parametrize("name", NAMES)
def test_full_size_final_output(name):
    wl = W.BY_NAME[name]
    g = load_golden(name)
    inp = W.make_inputs(wl)
    check_inputs(g, inp)
    say(f"[case] full-size {name} epilogue={W.EPI_NAMES[wl.epi]} x={wl.x_shape}")
    out, st, _ = run_gpu(wl, inp)
    assert np.isfinite(out).all()
    idx = g["sample_index"]
    if wl.epi == W.EPI_SCALE_BN_TRAIN_AVGPOOL:
        o2 = out.reshape(wl.n, wl.cout)
        assert max_err(o2, g["out"]) <= TOL
        np.testing.assert_allclose(st[:, 0], g["stats"][:, 0], rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(st[:, 1], g["stats"][:, 1], rtol=1e-5, atol=1e-6)
        # the batch mean of the pooled output is beta
        np.testing.assert_allclose(o2.astype(np.float64).mean(axis=0), inp.beta.astype(np.float64), atol=1e-5)
        return
    assert max_err(out[tuple(idx.T)], g["out_at_samples"]) <= TOL
    if wl.epi == W.EPI_RELU_GROUPNORM:
        np.testing.assert_allclose(st[..., 0], g["stats"][..., 0], rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(st[..., 1], g["stats"][..., 1], rtol=1e-5, atol=1e-6)
        # per (n, group): mean 0 and variance var/(var+eps) before the affine step
        ga = inp.gamma.astype(np.float64)[None, :, None]
        be = inp.beta.astype(np.float64)[None, :, None]
        z = (out.reshape(wl.n, wl.cout, -1).astype(np.float64) - be) / ga
        z = z.reshape(wl.n, wl.groups, -1)
        rstd = g["stats"][..., 1]
        var = 1.0 / rstd ** 2 - wl.eps
        np.testing.assert_allclose(z.mean(axis=2), 0.0, atol=2e-5)
        np.testing.assert_allclose(z.var(axis=2), var / (var + wl.eps), rtol=1e-4)
    if wl.epi == W.EPI_SOFTMAX_SIGMOID:
        # sigmoid of a probability lies in (0.5, sigmoid(1)]
        assert out.min() > 0.5 and out.max() <= 1.0 / (1.0 + np.exp(-1.0)) + 1e-6


@pytest.mark.parametrize("name", NAMES)
def test_full_size_raw_convolution(name):
    wl = W.BY_NAME[name]
    g = load_golden(name)
    inp = W.make_inputs(wl)
    say(f"[case] full-size raw conv {name} x={wl.x_shape}")
    raw, _, _ = run_gpu(wl.with_(epi=W.EPI_NONE), inp, kind=W.EPI_NONE, want_stats=False)
    idx = g["sample_index"]
    assert max_err(raw[tuple(idx.T)], g["raw_at_samples"]) <= TOL


@pytest.mark.parametrize("name", NAMES)
def test_full_size_tuned_plan(name):
    """The plan the benchmark times: convt3d_autotune on the full-size buffers
    (as bench.py calls it before its warm-up), then one fused call, checked at
    the golden's sampled voxels (gathered on the device) and on its statistics.
    Runs after the default-plan tests above: the tuned plan is kept for the
    rest of the process."""
    import torch
    from activation_epilogues_amd import convt3d as C
    from gpu_helpers import geom_of, to_dev
    wl = W.BY_NAME[name]
    g = load_golden(name)
    inp = W.make_inputs(wl)
    check_inputs(g, inp)
    say(f"[case] full-size tuned plan {name} x={wl.x_shape}")
    call = C.FusedCall(geom_of(wl), wl.epi, wl.groups, wl.eps, wl.scale, want_stats=True)
    x, w, b = to_dev(inp.x), to_dev(inp.w), to_dev(inp.b)
    gamma, beta = to_dev(inp.gamma), to_dev(inp.beta)
    call.prepack(w)
    res = call.autotune(x, b, gamma, beta)
    info = call.plan_info()
    say(f"  tuned: chosen {res['chosen']} of {res['candidates']}, plan {C.plan_string(info)} "
        f"phase_loop {info['phase_loop']}")
    assert info["tuned"] == 1
    call.out.fill_(float("nan"))
    if call.stats is not None:
        call.stats.fill_(float("nan"))
    out = call(x, b, gamma, beta)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    st = None if call.stats is None else call.stats.cpu().numpy()
    if wl.epi == W.EPI_SCALE_BN_TRAIN_AVGPOOL:
        o2 = out.reshape(wl.n, wl.cout).cpu().numpy()
        assert max_err(o2, g["out"]) <= TOL
        np.testing.assert_allclose(st[:, 0], g["stats"][:, 0], rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(st[:, 1], g["stats"][:, 1], rtol=1e-5, atol=1e-6)
        return
    idx = torch.from_numpy(np.ascontiguousarray(g["sample_index"])).to(out.device, torch.long)
    got = out[tuple(idx[:, i] for i in range(idx.shape[1]))].cpu().numpy()
    assert max_err(got, g["out_at_samples"]) <= TOL
    if wl.epi == W.EPI_RELU_GROUPNORM:
        np.testing.assert_allclose(st[..., 0], g["stats"][..., 0], rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(st[..., 1], g["stats"][..., 1], rtol=1e-5, atol=1e-6)
    if wl.epi == W.EPI_SOFTMAX_SIGMOID:
        assert float(out.min()) > 0.5 and float(out.max()) <= 1.0 / (1.0 + np.exp(-1.0)) + 1e-6


@pytest.mark.parametrize("name", [wl.name for wl in W.WORKLOADS] + ["k3s1_gn_g4_dl2", "k3s2_softmax_c256"])
def test_full_size_every_element_against_the_oracle(name):
    """Every element of the full-size output, and of the raw convolution, of
    every sample (so the per-sample offsets of all n samples are exercised),
    against the fp64 oracle on the same inputs: the plan the benchmark times
    (tuned above for these workloads; the tiny case runs its model plan)."""
    import oracle
    wl = W.BY_NAME[name]
    inp = W.make_inputs(wl)
    say(f"[case] full-size every element {name} x={wl.x_shape}")
    out, st, _ = run_gpu(wl, inp)
    raw, _, _ = run_gpu(wl.with_(epi=W.EPI_NONE), inp, kind=W.EPI_NONE, want_stats=False)
    ref = oracle.run_workload(wl, inp)
    err_out = max_err(out, ref.out.reshape(out.shape))
    err_raw = max_err(raw, ref.y.reshape(raw.shape))
    say(f"  max|err| final {err_out:.2e}, raw conv {err_raw:.2e}")
    assert err_out <= TOL and err_raw <= TOL
    if st is not None:
        np.testing.assert_allclose(st, ref.stats.reshape(st.shape), rtol=1e-5, atol=1e-6)
