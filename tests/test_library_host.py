"""Host-side checks of libconvt3d that need no GPU: the library loads, exports
every function include/convt3d.h declares, computes output sizes, workspace
sizes and plans, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from activation_epilogues_amd import convt3d as C
from activation_epilogues_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convt3d.h")

pytestmark = pytest.mark.skipif(not os.path.exists(C.LIB_PATH), reason="libconvt3d.so not built")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(convt3d_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def geom_of(wl, n=None):
    return C.make_geom(wl.n if n is None else n, wl.cin, wl.cout, wl.d, wl.h, wl.w, wl.k, wl.stride,
                       wl.pad, wl.out_pad, wl.dilation, wl.conv_groups)


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 8, names
    L = C.lib()  # through the binding: after torch's HIP runtime
    for nm in names:
        assert hasattr(L, nm), nm
    assert sorted(C.EXPORTED) == names


def test_general_geometry_dims_and_macs_match_brute_force():
    """Per-dim kernel / stride / pad / output padding, dilation and groups: the
    output size and the in-range multiply-add count the planner reports."""
    rng = np.random.default_rng(3)
    done = 0
    while done < 60:
        wl = W.random_general_geometry(rng, max_in=7)
        ks, ss, ps, ops, dls = (W.triple(v) for v in (wl.k, wl.stride, wl.pad, wl.out_pad, wl.dilation))
        od = [oracle.out_dim_general(n, *a) for n, a in zip((wl.d, wl.h, wl.w), zip(ks, ss, ps, ops, dls))]
        if min(od) <= 0:
            with pytest.raises(C.Convt3dError):
                C.convt3d_output_dims(geom_of(wl))
            continue
        assert C.convt3d_output_dims(geom_of(wl)) == tuple(od)
        per_dim = []
        for n_in, n_out, k, s, p, dl in zip((wl.d, wl.h, wl.w), od, ks, ss, ps, dls):
            per_dim.append(sum(0 <= s * i - p + dl * t < n_out for i in range(n_in) for t in range(k)))
        want = wl.n * (wl.cin // wl.conv_groups) * wl.cout * per_dim[0] * per_dim[1] * per_dim[2]
        info = C.convt3d_get_plan_info(geom_of(wl), C.make_epilogue(0))
        assert info["valid_macs"] == want
        assert info["issued_macs"] >= want
        assert C.convt3d_packed_weight_bytes(geom_of(wl)) >= 4 * wl.cin * (wl.cout // wl.conv_groups) * \
            ks[0] * ks[1] * ks[2]
        done += 1


def test_output_dims_match_oracle():
    for wl in W.WORKLOADS:
        assert C.convt3d_output_dims(geom_of(wl)) == oracle.out_dims(wl.d, wl.h, wl.w, wl.k, wl.stride,
                                                                   wl.pad, wl.out_pad)
    rng = np.random.default_rng(0)
    for _ in range(200):
        wl = W.random_geometry(rng, max_in=9)
        od = oracle.out_dims(wl.d, wl.h, wl.w, wl.k, wl.stride, wl.pad, wl.out_pad)
        if min(od) <= 0:
            with pytest.raises(C.Convt3dError):
                C.convt3d_output_dims(geom_of(wl))
        else:
            assert C.convt3d_output_dims(geom_of(wl)) == od


def test_status_strings():
    for st in range(11):
        assert C.status_string(st) != "unknown status"
    assert C.status_string(123) == "unknown status"


def test_plans_for_the_five_workloads():
    for wl in W.WORKLOADS:
        g = geom_of(wl)
        e = C.make_epilogue(wl.epi, wl.groups, wl.eps, wl.scale)
        info = C.convt3d_get_plan_info(g, e)
        assert info["valid_macs"] > 0
        assert info["issued_macs"] >= info["valid_macs"]
        assert info["lds_bytes"] <= 80 * 1024
        if wl.epi == W.EPI_SOFTMAX_SIGMOID:
            assert info["waves_co"] == 1 and info["co_blocks_per_wave"] * 32 >= wl.cout
        ws = C.convt3d_workspace_size(g, e)
        if wl.epi in (W.EPI_RELU_GROUPNORM, W.EPI_SCALE_BN_TRAIN_AVGPOOL):
            assert ws > 0
        assert C.convt3d_packed_weight_bytes(g) >= wl.cin * wl.cout * wl.k ** 3 * 4


def test_valid_mac_count_matches_brute_force_tap_count():
    rng = np.random.default_rng(1)
    for _ in range(30):
        wl = W.random_geometry(rng, max_in=7)
        if min(oracle.out_dims(wl.d, wl.h, wl.w, wl.k, wl.stride, wl.pad, wl.out_pad)) <= 0:
            continue
        od = oracle.out_dims(wl.d, wl.h, wl.w, wl.k, wl.stride, wl.pad, wl.out_pad)
        per_dim = []
        for n_in, n_out in zip((wl.d, wl.h, wl.w), od):
            cnt = 0
            for i in range(n_in):
                for t in range(wl.k):
                    o = wl.stride * i - wl.pad + t
                    cnt += 0 <= o < n_out
            per_dim.append(cnt)
        want = wl.n * wl.cin * wl.cout * per_dim[0] * per_dim[1] * per_dim[2]
        info = C.convt3d_get_plan_info(geom_of(wl), C.make_epilogue(0))
        assert info["valid_macs"] == want


FAKE = 0x100000  # never dereferenced: every case below fails its checks before any launch


@pytest.mark.parametrize("field,value,code", [
    ("n", -1, 2), ("cin", 0, 2), ("cout", 0, 2), ("d", 0, 2), ("k", 0, 2), ("stride", 0, 2),
    ("stride", 5, 2), ("pad", -1, 2), ("out_pad", 1, 2), ("dilation", 0, 2), ("groups", 0, 2),
    ("groups", 3, 2),
])
def test_bad_geometry_is_rejected(field, value, code):
    """Bad values, per-dim ones set along h only."""
    g = C.make_geom(1, 4, 8, 3, 3, 3, 3)
    if field in ("k", "stride", "pad", "out_pad", "dilation"):
        getattr(g, field)[1] = value
    else:
        setattr(g, field, value)
    e = C.make_epilogue(0)
    st = C.convt3d_fused(FAKE, FAKE, None, g, e, FAKE + (1 << 30), None, 0, stream=0, check=False)
    assert st == code
    assert C.convt3d_workspace_size(g, e) == 0


def test_empty_output_is_rejected():
    g = C.make_geom(1, 2, 2, 1, 1, 1, 3, 1, 2, 0)  # (1-1)*1 - 4 + 2 + 0 + 1 = -1
    st = C.convt3d_fused(FAKE, FAKE, None, g, C.make_epilogue(0), FAKE * 4, None, 0, stream=0, check=False)
    assert st == 2


def test_groups_and_epilogue_checks():
    g = C.make_geom(1, 4, 12, 3, 3, 3, 3)
    for groups in (0, 5, -2):
        st = C.convt3d_fused(FAKE, FAKE, None, g, C.make_epilogue(1, groups), FAKE * 64, FAKE * 128, 1 << 20,
                             stream=0, check=False)
        assert st == 3
    st = C.convt3d_fused(FAKE, FAKE, None, g, C.make_epilogue(7), FAKE * 64, None, 0, stream=0, check=False)
    assert st == 6
    st = C.convt3d_fused(FAKE, FAKE, None, g, C.make_epilogue(5), FAKE * 64, None, 0, stream=0, check=False)
    assert st == 6


def test_softmax_beyond_one_workgroup_runs_as_a_second_pass():
    """cout > 128 does not fit the in-register softmax: the plan stores y and
    finishes in a separate pass; cout <= 128 keeps the fused epilogue."""
    for cout, want in ((128, 0), (129, 1), (300, 1)):
        info = C.convt3d_get_plan_info(C.make_geom(2, 8, cout, 5, 6, 7, 3, 2, 1, 1), C.make_epilogue(2))
        assert info["softmax_pass"] == want
        if want:
            assert info["waves_co"] * info["co_blocks_per_wave"] >= 1  # a plain conv plan


def eval_bins_brute_force(wl):
    """Bins per dim of the eval-mode path: the input range cut wherever some
    tap starts or stops reaching the output (counted by brute force)."""
    od = oracle.out_dims(wl.d, wl.h, wl.w, wl.k, wl.stride, wl.pad, wl.out_pad)
    nb = []
    for n_in, n_out in zip((wl.d, wl.h, wl.w), od):
        cuts = {0, n_in}
        for t in range(wl.k):
            reach = [i for i in range(n_in) if 0 <= wl.stride * i - wl.pad + t < n_out]
            if reach:
                cuts.update((min(reach), max(reach) + 1))
        nb.append(len(cuts) - 1)
    return nb[0] * nb[1] * nb[2]


def test_eval_mode_bins_and_weight_size():
    rng = np.random.default_rng(5)
    seen = set()
    for _ in range(60):
        wl = W.random_geometry(rng, max_in=9)
        if min(oracle.out_dims(wl.d, wl.h, wl.w, wl.k, wl.stride, wl.pad, wl.out_pad)) <= 0:
            continue
        g = geom_of(wl)
        nb = eval_bins_brute_force(wl)
        info = C.convt3d_get_plan_info(g, C.make_epilogue(4))
        assert info["eval_bins"] == nb
        assert info["valid_macs"] == 0  # no convolution
        assert C.convt3d_eval_weight_bytes(g) == wl.cin * wl.cout * nb * 4
        assert C.convt3d_workspace_size(g, C.make_epilogue(4)) > 0
        seen.add(nb)
    assert 1 in seen and max(seen) > 8
    # the p77 shape (pad 0): one bin, the plain tap sum
    wl = W.BY_NAME["k5s1_bnpool_eval"]
    assert C.convt3d_get_plan_info(geom_of(wl), C.make_epilogue(4))["eval_bins"] == 1
    # kernels wider than 31 taps are not supported by the eval path
    big = C.make_geom(1, 2, 2, 3, 3, 3, 32)
    assert C.convt3d_eval_weight_bytes(big) == 0
    with pytest.raises(C.Convt3dError):
        C.convt3d_get_plan_info(big, C.make_epilogue(4))


def test_pointer_checks():
    g = C.make_geom(1, 4, 8, 3, 3, 3, 3)
    e_none = C.make_epilogue(0)
    out = FAKE * 64
    assert C.convt3d_fused(None, FAKE, None, g, e_none, out, None, 0, stream=0, check=False) == 1
    assert C.convt3d_fused(FAKE, None, None, g, e_none, out, None, 0, stream=0, check=False) == 1
    assert C.convt3d_fused(FAKE, FAKE, None, g, e_none, None, None, 0, stream=0, check=False) == 1
    assert C.convt3d_fused(FAKE + 4, FAKE, None, g, e_none, out, None, 0, stream=0, check=False) == 4
    assert C.convt3d_fused(FAKE, FAKE, FAKE + 8, g, e_none, out, None, 0, stream=0, check=False) == 4
    # out overlapping x
    assert C.convt3d_fused(FAKE, FAKE * 2, None, g, e_none, FAKE + 64, None, 0, stream=0, check=False) == 9
    e_gn = C.make_epilogue(1, 2)
    need = C.convt3d_workspace_size(g, e_gn)
    assert need > 0
    assert C.convt3d_fused(FAKE, FAKE, None, g, e_gn, out, None, need, stream=0, check=False) == 5
    assert C.convt3d_fused(FAKE, FAKE, None, g, e_gn, out, FAKE * 128, need - 1, stream=0, check=False) == 5
    assert C.convt3d_prepack_weights(g, None, FAKE, stream=0, check=False) == 1
    assert C.convt3d_prepack_weights(g, FAKE, FAKE + 4, stream=0, check=False) == 4


def test_running_statistics_checks():
    """Both running buffers or none; the unbiased update needs more than one
    value per channel."""
    g = C.make_geom(1, 4, 8, 3, 3, 3, 3)
    need = C.convt3d_workspace_size(g, C.make_epilogue(3))
    e = C.make_epilogue(3, running_mean=FAKE * 256)
    assert C.convt3d_fused(FAKE, FAKE, None, g, e, FAKE * 64, FAKE * 128, need, stream=0, check=False) == 1
    one = C.make_geom(1, 4, 8, 1, 1, 1, 1)  # one output voxel, one sample
    e = C.make_epilogue(3, running_mean=FAKE * 256, running_var=FAKE * 260)
    need = C.convt3d_workspace_size(one, e)
    assert C.convt3d_fused(FAKE, FAKE, None, one, e, FAKE * 64, FAKE * 128, need, stream=0, check=False) == 6


def test_epilogue_only_argument_checks():
    n, c, S = 2, 8, 60
    y, out, ws = FAKE, FAKE * 64, FAKE * 128
    gn = C.make_epilogue(1, 4)
    need = C.convt3d_epilogue_workspace_size(n, c, S, gn)
    assert need >= n * c * 2 * 4 * 2
    assert C.convt3d_epilogue_workspace_size(n, c, S, C.make_epilogue(2)) == 0
    only = lambda *a: C.convt3d_epilogue_only(*a, stream=0, check=False)
    assert only(None, n, c, S, gn, out, ws, need) == 1
    assert only(y, n, c, S, gn, None, ws, need) == 1
    assert only(y, n, c, S, C.make_epilogue(0), out, ws, need) == 6
    assert only(y, n, c, S, C.make_epilogue(9), out, ws, need) == 6
    assert only(y, n, c, S, C.make_epilogue(1, 3), out, ws, need) == 3
    assert only(y, -1, c, S, gn, out, ws, need) == 2
    assert only(y, n, 0, S, gn, out, ws, need) == 2
    assert only(y, n, c, 0, gn, out, ws, need) == 2
    assert only(y + 4, n, c, S, gn, out, ws, need) == 4
    assert only(y, n, c, S, gn, y + 16, ws, need) == 9          # partial overlap
    assert only(y, n, c, S, C.make_epilogue(3), y, ws, need) == 9  # pooled output over y
    assert only(y, n, c, S, gn, out, ws, need - 1) == 5
    assert only(y, n, c, S, gn, out, None, need) == 5
    bn = C.make_epilogue(3, running_var=FAKE * 512)
    assert only(y, n, c, S, bn, out, ws, need) == 1
    bn = C.make_epilogue(3, running_mean=FAKE * 256, running_var=FAKE * 512)
    assert only(y, 1, c, 1, bn, out, ws, need) == 6
    assert only(y, 1 << 20, 1 << 10, 1 << 10, gn, out, ws, need) == 8
    # an empty batch launches nothing
    assert only(y, 0, c, S, gn, out, ws, need) == 0


def test_size_limits():
    """Sizes past the 32-bit offsets the kernels use are refused with
    CONVT3D_ERR_TOO_LARGE before anything runs; just inside, a plan exists."""
    def status(g, kind=0):
        try:
            C.convt3d_get_plan_info(g, C.make_epilogue(kind))
            return 0
        except C.Convt3dError as ex:
            return ex.status
    # per-channel output size: the conv kernel's row byte offsets reach 20 * S
    assert status(C.make_geom(1, 2, 2, 590, 590, 590, 3, 1, 1, 0)) == 0      # S = 590^3, 20 S < 2^32
    assert status(C.make_geom(1, 2, 2, 600, 600, 600, 3, 1, 1, 0)) == 8      # S = 600^3, 20 S > 2^32
    # whole output and whole input beyond 2^31 elements
    assert status(C.make_geom(11, 1, 1, 590, 590, 590, 1)) == 8              # 11 * 590^3 > 2^31
    assert status(C.make_geom(1, 11, 1, 590, 590, 590, 1)) == 8
    # input channel planes: the halo staging's 32-bit buffer offsets reach
    # 2^29 voxels (k = 1 with a large pad keeps the output small)
    assert status(C.make_geom(1, 1, 1, 1024, 1024, 512, 1, 1, (250, 250, 200))) == 0   # 2^29 voxels
    assert status(C.make_geom(1, 1, 1, 1024, 1024, 513, 1, 1, (250, 250, 200))) == 8   # past 2^29
    # packed weights
    assert status(C.make_geom(1, 1024, 1024, 2, 2, 2, 16)) == 8
    assert C.convt3d_packed_weight_bytes(C.make_geom(1, 1024, 1024, 2, 2, 2, 16)) == 0


def test_empty_batch_is_a_no_op():
    g = C.make_geom(0, 4, 8, 3, 3, 3, 3)
    for kind in (0, 1, 2, 3, 4):
        e = C.make_epilogue(kind, 2)
        # null pointers are fine: nothing is launched for an empty batch
        assert C.convt3d_fused(None, None, None, g, e, None, None, 0, stream=0, check=False) == 0


def test_autotune_argument_checks():
    """convt3d_autotune checks its arguments like convt3d_fused before timing anything."""
    g = C.make_geom(1, 4, 8, 3, 3, 3, 3)
    e = C.make_epilogue(0)
    out = FAKE * 64
    lib = C.lib()
    res = C.TuneResult()

    def tune(x, wp, bias, out_, ws, ws_bytes, geom=g, epi=e):
        return lib.convt3d_autotune(x, wp, bias, ctypes.byref(geom), ctypes.byref(epi), out_, ws, ws_bytes, 0,
                                    ctypes.byref(res))

    assert tune(None, FAKE, None, out, None, 0) == 1
    assert tune(FAKE, None, None, out, None, 0) == 1
    assert tune(FAKE + 4, FAKE, None, out, None, 0) == 4
    assert tune(FAKE, FAKE * 2, None, FAKE + 64, None, 0) == 9
    # an empty batch times nothing and succeeds with null buffers
    g0 = C.make_geom(0, 4, 8, 3, 3, 3, 3)
    assert tune(None, None, None, None, None, 0, geom=g0) == 0
    assert res.candidates == 0



def test_plan_string_selects_the_same_plan(monkeypatch):
    """The CONVT3D_PLAN string a plan reports forces that plan again."""
    for wl in W.WORKLOADS:
        e = C.make_epilogue(wl.epi, wl.groups)
        monkeypatch.delenv("CONVT3D_PLAN", raising=False)
        monkeypatch.delenv("CONVT3D_PHASE_LOOP", raising=False)
        info = C.convt3d_get_plan_info(geom_of(wl), e)
        monkeypatch.setenv("CONVT3D_PLAN", C.plan_string(info))
        monkeypatch.setenv("CONVT3D_PHASE_LOOP", str(info["phase_loop"]))
        again = C.convt3d_get_plan_info(geom_of(wl), e)
        assert again == info, wl.name


@pytest.mark.parametrize("name,margin", [("k3s1_gn", 0.96), ("k5s1_bnpool", 0.99)])
def test_one_border_tiled_with_the_interior_cuts_padding(monkeypatch, name, margin):
    """k3 over 32 inputs gives 34 outputs per dim and k5 over 16 or 32 gives 20
    or 36: a 2 + 32 (4 + 16, 4 + 32) segmentation lets the boxes divide the long
    segment, where low border / interior / high border leaves an interior of
    30 (12, 28) that they do not.  The plan keeps one border inside the
    interior (border_split bit 3 + d or 6 + d) and issues fewer MACs than the
    same variant and wave grid with every border on its own.  (The BatchNorm-
    pool epilogue stores no y, so its border boxes may be narrower than 16 and
    the three-way split loses less there.)"""
    wl = W.BY_NAME[name]
    e = C.make_epilogue(wl.epi, wl.groups, wl.eps, wl.scale)
    monkeypatch.delenv("CONVT3D_PLAN", raising=False)
    monkeypatch.delenv("CONVT3D_PHASE_LOOP", raising=False)
    info = C.convt3d_get_plan_info(geom_of(wl), e)
    assert info["border_split"] >> 3, info["border_split"]
    monkeypatch.setenv("CONVT3D_PLAN", f"{info['variant']},{info['waves_co']},-1,-1,-1,-1,7")
    monkeypatch.setenv("CONVT3D_PHASE_LOOP", str(info["phase_loop"]))
    three = C.convt3d_get_plan_info(geom_of(wl), e)
    assert three["border_split"] == 7
    assert three["valid_macs"] == info["valid_macs"]
    assert info["issued_macs"] < margin * three["issued_macs"]


def test_sigmoid_polynomial_matches_its_generator():
    """The softmax epilogues' sigmoid coefficients (one table, shared by the
    fused and the standalone kernels) are the ones sigmoid_poly.py derives, and
    their float32 evaluation 1/2 + p R(p^2) stays within 1.2e-7 (two units in
    the last place of a result in [0.5, 0.74]) of the definition on [0, 1]."""
    import importlib.util
    csrc = os.path.join(ROOT, "activation_epilogues_amd", "csrc")
    spec = importlib.util.spec_from_file_location("sigmoid_poly", os.path.join(csrc, "sigmoid_poly.py"))
    sp = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(sp)
    want = sp.coefficients()
    src = open(os.path.join(csrc, "convt3d_internal.hpp")).read()
    m = re.search(r"kSigmoidOdd\[4\]\s*=\s*\{([^}]*)\}", src)
    assert m
    got = np.array([float(t.strip().rstrip("f")) for t in m.group(1).split(",")], dtype=np.float32)
    assert np.array_equal(got, want)
    p = np.linspace(0.0, 1.0, 100001).astype(np.float32)
    err = np.abs(sp.eval32(got, p).astype(np.float64) - 1.0 / (1.0 + np.exp(-p.astype(np.float64)))).max()
    assert err < 1.2e-7


def test_plan_cache_keys_on_every_override(monkeypatch):
    """A plan cached for a geometry is not reused under a different phase-loop or
    work-order override (the overrides are part of the cache key)."""
    g = C.make_geom(2, 20, 40, 7, 9, 11, 3, 2, 1, 1)
    e = C.make_epilogue(1, 4)
    monkeypatch.delenv("CONVT3D_PLAN", raising=False)
    monkeypatch.setenv("CONVT3D_PHASE_LOOP", "0")
    assert C.convt3d_get_plan_info(g, e)["phase_loop"] == 0
    monkeypatch.setenv("CONVT3D_PHASE_LOOP", "1")
    assert C.convt3d_get_plan_info(g, e)["phase_loop"] == 1
    monkeypatch.delenv("CONVT3D_PHASE_LOOP")
    monkeypatch.setenv("CONVT3D_ORDER", "0")
    assert C.convt3d_get_plan_info(g, e)["xcd_order"] == 0
    monkeypatch.setenv("CONVT3D_ORDER", "1")
    assert C.convt3d_get_plan_info(g, e)["xcd_order"] == 1

PREFETCH_VARIANT = 15  # the register-prefetch build in the library's variant table


def test_prefetch_build_needs_a_second_chunk(monkeypatch):
    """The register-prefetch kernel takes one octet of input channels per
    chunk and needs a further chunk to prefetch: forced on a layer with one
    octet it has no plan; with two it runs 8-channel chunks."""
    monkeypatch.setenv("CONVT3D_PLAN", f"{PREFETCH_VARIANT},-1,-1,-1,-1,-1")
    monkeypatch.setenv("CONVT3D_PHASE_LOOP", "0")
    e = C.make_epilogue(1, 4)
    with pytest.raises(C.Convt3dError):
        C.convt3d_get_plan_info(C.make_geom(2, 8, 32, 6, 6, 6, 3), e)
    info = C.convt3d_get_plan_info(C.make_geom(2, 16, 32, 6, 6, 6, 3), e)
    assert (info["variant"], info["ci_chunk"], info["pos_blocks_per_wave"]) == (PREFETCH_VARIANT, 8, 4)


def test_profile_kind_mask_is_checked():
    """convt3d_profile_begin_kinds takes a nonzero subset of the kernel kinds;
    a session with nothing recorded ends with every duration 0."""
    lib = C.lib()
    assert lib.convt3d_profile_begin_kinds(0) == 6
    assert lib.convt3d_profile_begin_kinds(0x20) == 6
    assert lib.convt3d_profile_begin_kinds(0xFFFFFFFF) == 6
    for mask in (C.PROFILE_CONV, C.PROFILE_REDUCE | C.PROFILE_PREPACK, C.PROFILE_ALL):
        C.convt3d_profile_begin_kinds(mask)
        prof = C.convt3d_profile_end()
        assert prof["calls"] == 0
        assert all(prof[k] == 0.0 for k in ("conv_ms", "finalize_ms", "normalize_ms", "reduce_ms", "prepack_ms"))
    assert lib.convt3d_profile_begin() == 0
    assert C.convt3d_profile_end()["calls"] == 0


def test_library_binds_to_the_hip_runtime_torch_loads():
    """Loading the library first must not leave two HIP runtimes in the process:
    the binding imports torch before the library, so the library binds to
    torch's runtime (which owns the caller's memory and streams)."""
    import subprocess
    import sys
    code = ("from activation_epilogues_amd import convt3d as C\n"
            "C.lib()\n"
            "import torch\n"
            "print('|'.join(C._hip_runtimes()))\n")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    rts = res.stdout.strip().splitlines()[-1].split("|")
    assert len(rts) == 1, rts
    import torch
    assert os.path.dirname(rts[0]) == os.path.join(os.path.dirname(torch.__file__), "lib"), rts
