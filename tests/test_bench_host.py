"""Host-side checks of bench.py's reading of the committed rocprofv3 traffic
summaries: a summary counts only while the kernel source it was taken from is
unchanged, and the plan it was taken on is reported with it."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _write_summary(path, sha, plan, nbytes):
    with open(path, "w") as f:
        f.write("# HBM traffic of convt3d_mfma_kernel, workload demo\n")
        f.write(f"# command: rocprofv3 --pmc FETCH_SIZE -- python3 bench.py --workload demo --plan {plan} "
                "--phase-loop 0\n")
        f.write(f"kernel_source_sha256_16: {sha}\n")
        f.write(f"hbm_bytes_per_launch: {nbytes}\n")


def test_traffic_counts_only_for_the_current_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    path = tmp_path / "convt3d_mfma_kernel_demo_traffic.txt"
    _write_summary(path, bench.kernel_source_hash(), "1,4,2,2,32,16,103", 12345)
    assert bench.stored_traffic("demo") == (12345.0, "1,4,2,2,32,16,103")
    _write_summary(path, "0" * 16, "1,4,2,2,32,16,103", 12345)
    assert bench.stored_traffic("demo") == (None, None)
    assert bench.stored_traffic("missing") == (None, None)


def test_committed_summaries_parse():
    for name in os.listdir(bench.PROFILES):
        if not name.endswith("_traffic.txt"):
            continue
        kernel = "eval_binsum_kernel" if name.startswith("eval_binsum_kernel") else "convt3d_mfma_kernel"
        workload = name[len(kernel) + 1:-len("_traffic.txt")]
        nbytes, plan = bench.stored_traffic(workload, kernel)
        # taken from the current source: a byte count; conv summaries name their plan
        assert nbytes is None or nbytes > 0
        if nbytes is not None and kernel == "convt3d_mfma_kernel":
            assert plan is not None and plan.count(",") == 6


def test_more_than_one_gpu_exits_with_a_message():
    """--gpus N > 1 stops before touching a GPU, with a status of 2 and a message."""
    import subprocess
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""
