"""Every compiled kernel instantiation against the fp64 oracle.

The planner normally picks one configuration per geometry, so most kernel
variants only run when their shape wins.  Here each variant (and each
phase-group-loop build) is forced through CONVT3D_PLAN / CONVT3D_PHASE_LOOP on
a ragged geometry (Cin = 20: a partial channel octet and several chunks; odd
sizes; border tiles), and strides 3 and 4 get cases of their own."""
import numpy as np
import pytest

import oracle
from activation_epilogues_amd import workloads as W

from gpu_helpers import TOL, geom_of, max_err, say, to_dev

pytestmark = pytest.mark.gpu

# (co blocks, w-phases, position blocks per wave, softmax epilogue, has a
# phase-group-loop build) in the library's variant order
VARIANTS = [
    (1, 1, 8, False, False), (1, 1, 4, False, True), (1, 1, 2, False, False),
    (1, 2, 4, False, True), (1, 2, 2, False, True),
    (1, 1, 4, True, False), (1, 1, 2, True, True), (1, 2, 2, True, True),
    (2, 1, 4, True, False), (2, 2, 2, True, True), (2, 1, 2, True, True), (2, 2, 1, True, True),
    (4, 1, 2, True, False), (4, 2, 1, True, True), (4, 1, 1, True, True),
    (1, 1, 4, False, False),  # the register-prefetch build of the next channel chunk
]
CASES = [(vi, 0) for vi in range(len(VARIANTS))] + [(vi, 1) for vi, v in enumerate(VARIANTS) if v[4]]


def case_workload(vi, ploop, epi_cycle):
    cbw, nph, pbw, sm, _ = VARIANTS[vi]
    stride = 2 if (nph == 2 or ploop) else 1
    if sm:
        epi = W.EPI_SOFTMAX_SIGMOID
        cout = {1: 24, 2: 56, 4: 100}[cbw]
    else:
        epi = [W.EPI_RELU_GROUPNORM, W.EPI_NONE, W.EPI_SCALE_BN_TRAIN_AVGPOOL][epi_cycle % 3]
        cout = 40
    return W.Workload(f"v{vi}pl{ploop}", 2, 20, cout, 7, 9, 11, k=3, stride=stride,
                      pad=1 if stride > 1 else 0, out_pad=1 if stride > 1 else 0, bias=True, epi=epi,
                      groups=4 if epi == W.EPI_RELU_GROUPNORM else 1, scale=2.0, seed=7000 + 10 * vi + ploop)


def run_and_check(wl):
    import torch
    from activation_epilogues_amd import convt3d as C
    inp = W.make_inputs(wl)
    call = C.FusedCall(geom_of(wl), wl.epi, wl.groups, wl.eps, wl.scale, want_stats=True)
    info = call.plan_info()
    x, w, b = to_dev(inp.x), to_dev(inp.w), to_dev(inp.b)
    gamma, beta = to_dev(inp.gamma), to_dev(inp.beta)
    call.prepack(w)
    call.out.fill_(float("nan"))
    out = call(x, b, gamma, beta)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ref = oracle.run_workload(wl, inp)
    err = max_err(out, ref.out.reshape(out.shape))
    assert err <= TOL, f"max|err| {err:.3e}"
    if call.stats is not None:
        st = call.stats.cpu().numpy()
        np.testing.assert_allclose(st, ref.stats.reshape(st.shape), rtol=1e-5, atol=1e-6)
    return info


@pytest.mark.parametrize("vi,ploop", CASES, ids=[f"v{vi}-pl{p}" for vi, p in CASES])
def test_forced_variant_matches_oracle(vi, ploop, monkeypatch):
    from activation_epilogues_amd import convt3d as C
    wl = case_workload(vi, ploop, vi)
    monkeypatch.setenv("CONVT3D_PLAN", f"{vi},-1,-1,-1,-1,-1")
    monkeypatch.setenv("CONVT3D_PHASE_LOOP", str(ploop))
    say(f"[case] variant {vi} phase_loop {ploop} epi {W.EPI_NAMES[wl.epi]} cout {wl.cout} s {wl.stride}")
    info = C.convt3d_get_plan_info(geom_of(wl), C.make_epilogue(wl.epi, wl.groups))
    cbw, nph, pbw = VARIANTS[vi][:3]
    assert (info["variant"], info["co_blocks_per_wave"], info["w_phases_per_wave"],
            info["pos_blocks_per_wave"], info["phase_loop"]) == (vi, cbw, nph, pbw, ploop)
    run_and_check(wl)


@pytest.mark.parametrize("stride,k,pad,out_pad,epi", [
    (3, 3, 1, 2, W.EPI_RELU_GROUPNORM), (3, 5, 2, 1, W.EPI_SOFTMAX_SIGMOID),
    (4, 4, 0, 3, W.EPI_NONE), (4, 6, 1, 0, W.EPI_SCALE_BN_TRAIN_AVGPOOL), (4, 3, 2, 1, W.EPI_SOFTMAX_SIGMOID),
])
def test_large_strides(stride, k, pad, out_pad, epi):
    wl = W.Workload(f"s{stride}k{k}", 2, 13, 40 if epi != W.EPI_SOFTMAX_SIGMOID else 48, 5, 6, 7, k=k,
                    stride=stride, pad=pad, out_pad=out_pad, bias=True, epi=epi,
                    groups=8 if epi == W.EPI_RELU_GROUPNORM else 1, scale=-0.5, seed=9100 + 10 * stride + k)
    say(f"[case] stride {stride} k {k} p {pad} op {out_pad} epi {W.EPI_NAMES[epi]}")
    run_and_check(wl)


# border segmentations (bit d: dim d split; bit 3 + d: low border alone, high
# border tiled with the interior; bit 6 + d: the reverse), each forced on
# geometries where every dim has both borders
SPLITS = [0, 7, 63, 455, 143, 103, 1, 260]


def border_workload(k, stride, split):
    """Geometry on which every dim has both borders and an interior, with the
    epilogue cycling over GroupNorm, BatchNorm and none."""
    epi = [W.EPI_RELU_GROUPNORM, W.EPI_SCALE_BN_TRAIN_AVGPOOL, W.EPI_NONE][SPLITS.index(split) % 3]
    return W.Workload(f"seg{split}k{k}s{stride}", 2, 16, 64, 10, 12, 14, k=k, stride=stride, pad=0, out_pad=0,
                      bias=True, epi=epi, groups=8 if epi == W.EPI_RELU_GROUPNORM else 1, scale=2.0,
                      seed=9100 + split + 10 * k)


@pytest.mark.parametrize("k,stride", [(3, 1), (4, 2), (5, 1)])
@pytest.mark.parametrize("split", SPLITS)
def test_forced_border_segmentation_matches_oracle(k, stride, split, monkeypatch):
    from activation_epilogues_amd import convt3d as C
    wl = border_workload(k, stride, split)
    e = C.make_epilogue(wl.epi, wl.groups)
    base = C.convt3d_get_plan_info(geom_of(wl), e)
    monkeypatch.setenv("CONVT3D_PLAN", f"{base['variant']},{base['waves_co']},-1,-1,-1,-1,{split}")
    monkeypatch.setenv("CONVT3D_PHASE_LOOP", str(base["phase_loop"]))
    info = C.convt3d_get_plan_info(geom_of(wl), e)
    say(f"[case] border split {split} k {k} s {stride} epi {W.EPI_NAMES[wl.epi]} plan {C.plan_string(info)}")
    assert info["border_split"] == split
    run_and_check(wl)


def test_prefetch_build_on_a_grouped_dilated_layer(monkeypatch):
    """The register-prefetch build on the shape it is for: four channel groups
    of 16 input channels (two chunks each), dilation 2, ragged sizes."""
    from activation_epilogues_amd import convt3d as C
    wl = W.Workload("rp_g4_dl2", 2, 64, 128, 9, 10, 11, k=3, dilation=2, conv_groups=4, bias=False,
                    epi=W.EPI_RELU_GROUPNORM, groups=8, seed=7400)
    monkeypatch.setenv("CONVT3D_PLAN", f"{len(VARIANTS) - 1},-1,-1,-1,-1,-1")
    monkeypatch.setenv("CONVT3D_PHASE_LOOP", "0")
    info = C.convt3d_get_plan_info(geom_of(wl), C.make_epilogue(wl.epi, wl.groups))
    say(f"[case] prefetch build, grouped dilated layer, plan {C.plan_string(info)}")
    assert info["variant"] == len(VARIANTS) - 1 and info["ci_chunk"] == 8
    run_and_check(wl)
