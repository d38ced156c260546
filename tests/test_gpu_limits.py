"""GPU parity at the largest per-channel output the conv kernel addresses:
S = 590^3 voxels, whose per-row byte offsets reach 20*S = 4.1e9, just below
2^32 (the planner refuses larger S).  The outputs are checked at sampled
voxels against the oracle's gather-form point evaluation (the whole oracle
would take minutes at this size)."""
import numpy as np
import pytest

import oracle
from activation_epilogues_amd import workloads as W

from gpu_helpers import TOL, run_gpu, say

pytestmark = pytest.mark.gpu

BIG = W.Workload("max_offsets", 1, 2, 2, 590, 590, 590, k=3, stride=1, pad=1, bias=True, epi=W.EPI_NONE,
                 seed=7700)


def sample_points(rng, dims, count):
    pts = [tuple(int(rng.integers(0, d)) for d in dims) for _ in range(count)]
    # the first and last voxels, where the offsets are smallest and largest
    pts += [(0, 0, 0), tuple(d - 1 for d in dims)]
    return pts


@pytest.mark.parametrize("kind", [W.EPI_NONE, W.EPI_SOFTMAX_SIGMOID])
def test_largest_channel_size(kind):
    wl = BIG.with_(epi=kind)
    say(f"[case] max offsets kind={kind} n=1 cin=2 cout=2 in=590^3 k3 p1")
    inp = W.make_inputs(wl)
    out, _, _ = run_gpu(wl, inp, kind, want_stats=False)
    assert out.shape == (1, 2, 590, 590, 590)
    rng = np.random.default_rng(7701)
    worst = 0.0
    for od, oh, ow in sample_points(rng, (590, 590, 590), 300):
        y = np.array([oracle.convt3d_point(inp.x, inp.w, inp.b, 1, 1, 0, 0, co, od, oh, ow) for co in range(2)])
        if kind == W.EPI_SOFTMAX_SIGMOID:
            want, _ = oracle.softmax_sigmoid(y.reshape(1, 2, 1, 1, 1))
            want = want.reshape(2)
        else:
            want = y
        worst = max(worst, float(np.abs(out[0, :, od, oh, ow].astype(np.float64) - want).max()))
    say(f"[case] max offsets kind={kind}: sampled max|err| {worst:.2e}")
    assert worst <= TOL
