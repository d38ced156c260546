"""CPU replay of the convolution kernel's address arithmetic, and the host
code under AddressSanitizer / UndefinedBehaviorSanitizer.

tests/replay/conv_replay.cpp links the library's planner and C ABI as they
are and replaces each kernel launch by a walk over every workgroup, wave and
lane of the grid, computing each address with the index functions the
kernel itself calls (csrc/conv_index.hpp).  It checks LDS reads and writes
against the workgroup's allocation (and that no LDS word is read before it
was cleared or staged), global reads against x / the packed weights / bias,
that every output and statistics partial is written exactly once, and that
the statistics merges read only partials the conv wrote.  The whole harness
is built with -fsanitize=address,undefined, so the planner's region tables,
the plan cache and the argument checks run under the sanitizers.

Cases: every kernel variant forced as the GPU variant test forces it, the
strides 3 and 4 cases, every forced border segmentation, random general
geometries (per-dim sizes, dilation, groups) of every epilogue, and the
named workloads at full size (the plan convt3d_fused runs)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from activation_epilogues_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "activation_epilogues_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "replay", "conv_replay.cpp")


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are missing")
    exe = str(tmp_path_factory.mktemp("replay") / "conv_replay")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-I", "/opt/rocm/include", os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "api.cpp"), SRC,
           "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    return exe


@pytest.fixture(scope="module")
def harness_tsan(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are missing")
    exe = str(tmp_path_factory.mktemp("replay_tsan") / "conv_replay_tsan")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-fno-omit-frame-pointer", "-pthread",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", "/opt/rocm/include",
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "api.cpp"), SRC, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    return exe


def case_line(name, wl, plan_env="-", ploop_env="-", mode="full"):
    t = W.triple
    k, s, p, op, dl = (t(v) for v in (wl.k, wl.stride, wl.pad, wl.out_pad, wl.dilation))
    nums = [wl.n, wl.cin, wl.cout, wl.d, wl.h, wl.w, *k, *s, *p, *op, *dl, wl.conv_groups, wl.epi, wl.groups]
    return " ".join([name] + [str(v) for v in nums] + [plan_env, ploop_env, mode])


def run(harness, lines, timeout=600):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("CONVT3D_PLAN", None)
    env.pop("CONVT3D_PHASE_LOOP", None)
    res = subprocess.run([harness], input="\n".join(lines) + "\n", capture_output=True, text=True, timeout=timeout,
                         env=env)
    out = res.stdout
    assert "ERROR: AddressSanitizer" not in res.stderr, res.stderr[-4000:]
    assert "runtime error" not in res.stderr, res.stderr[-4000:]
    assert res.returncode == 0, out[-4000:] + res.stderr[-2000:]
    oks = [ln for ln in out.splitlines() if ln.startswith("ok ")]
    assert len(oks) == len(lines), out[-4000:]
    return oks


def geom_of(wl):
    from activation_epilogues_amd import convt3d as C
    return C.make_geom(wl.n, wl.cin, wl.cout, wl.d, wl.h, wl.w, wl.k, wl.stride, wl.pad, wl.out_pad,
                       wl.dilation, wl.conv_groups)


def test_forced_variants_and_large_strides(harness):
    from test_gpu_variants import CASES, case_workload
    lines = [case_line(f"v{vi}pl{pl}", case_workload(vi, pl, vi), f"{vi},-1,-1,-1,-1,-1", str(pl))
             for vi, pl in CASES]
    for stride, k, pad, out_pad, epi in [(3, 3, 1, 2, W.EPI_RELU_GROUPNORM), (3, 5, 2, 1, W.EPI_SOFTMAX_SIGMOID),
                                         (4, 4, 0, 3, W.EPI_NONE), (4, 6, 1, 0, W.EPI_SCALE_BN_TRAIN_AVGPOOL),
                                         (4, 3, 2, 1, W.EPI_SOFTMAX_SIGMOID)]:
        wl = W.Workload(f"s{stride}k{k}", 2, 13, 40 if epi != W.EPI_SOFTMAX_SIGMOID else 48, 5, 6, 7, k=k,
                        stride=stride, pad=pad, out_pad=out_pad, bias=True, epi=epi,
                        groups=8 if epi == W.EPI_RELU_GROUPNORM else 1, scale=-0.5)
        lines.append(case_line(wl.name, wl))
    run(harness, lines)


def test_forced_border_segmentations(harness):
    """The plans test_gpu_variants forces: the model's kernel configuration
    with each border segmentation of every dim."""
    from activation_epilogues_amd import convt3d as C
    from test_gpu_variants import SPLITS, border_workload
    lines = []
    for k, stride in [(3, 1), (4, 2), (5, 1)]:
        for split in SPLITS:
            wl = border_workload(k, stride, split)
            base = C.convt3d_get_plan_info(geom_of(wl), C.make_epilogue(wl.epi, wl.groups))
            lines.append(case_line(wl.name, wl, f"{base['variant']},{base['waves_co']},-1,-1,-1,-1,{split}",
                                   str(base["phase_loop"])))
    oks = run(harness, lines)
    for ln, split in zip(oks, SPLITS * 3):
        assert f",{split} ploop" in ln, ln  # the forced segmentation is the one replayed


def test_random_general_geometries(harness):
    rng = np.random.default_rng(20261)
    lines = []
    epis = [W.EPI_NONE, W.EPI_RELU_GROUPNORM, W.EPI_SOFTMAX_SIGMOID, W.EPI_SCALE_BN_TRAIN_AVGPOOL]
    while len(lines) < 48:
        epi = epis[len(lines) % 4]
        wl = W.random_general_geometry(rng, max_in=7, max_ch=40, epi=epi)
        if epi == W.EPI_SCALE_BN_TRAIN_AVGPOOL and wl.n * wl.d * wl.h * wl.w < 2:
            continue
        from activation_epilogues_amd import convt3d as C
        try:
            C.convt3d_output_dims(geom_of(wl))
        except C.Convt3dError:
            continue
        lines.append(case_line(f"r{len(lines)}", wl))
    run(harness, lines)


def test_named_workloads_full_size(harness):
    """The plan convt3d_fused runs on each named workload at its full size
    (address ranges per wave; the border segmentations and candidates of the
    tuner are covered by the small cases above)."""
    lines = [case_line(wl.name, wl, mode="one") for wl in W.WORKLOADS + W.EXTRA_WORKLOADS]
    run(harness, lines, timeout=900)


def test_concurrent_planning_under_thread_sanitizer(harness_tsan):
    """Eight host threads plan the named workloads and random general
    geometries at once (each geometry first planned by whichever thread gets
    there), under ThreadSanitizer: no data race is reported, and every thread's
    plan, workspace and output sizes equal a serial lookup afterwards."""
    rng = np.random.default_rng(4242)
    lines = [case_line(wl.name, wl) for wl in W.WORKLOADS + W.EXTRA_WORKLOADS]
    while len(lines) < 24:
        wl = W.random_general_geometry(rng, max_in=7, max_ch=40, epi=len(lines) % 4)
        lines.append(case_line(f"r{len(lines)}", wl))
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 second_deadlock_stack=1")
    env.pop("CONVT3D_PLAN", None)
    env.pop("CONVT3D_PHASE_LOOP", None)
    res = subprocess.run([harness_tsan, "threads", "8"], input="\n".join(lines) + "\n", capture_output=True,
                         text=True, timeout=600, env=env)
    assert "WARNING: ThreadSanitizer" not in res.stderr, res.stderr[-6000:]
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "0 mismatches" in res.stdout, res.stdout[-2000:]
