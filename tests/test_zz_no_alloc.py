"""convt3d_fused_noalloc, the entry point that takes no workspace (the
library's static device scratch stands in for it), against convt3d_fused with
a caller workspace: same plan, same kernels, so bitwise the same outputs and
statistics, both within the tolerance of the fp64 oracle.  Calls follow one
another on the shared scratch, each later one smaller than the one before, so
a call that read what an earlier call left in the scratch would show."""
import numpy as np
import pytest

import oracle
from activation_epilogues_amd import workloads as W

from gpu_helpers import TOL, geom_of, max_err, say, to_dev

# (n, cin, cout, d, h, w, k, stride, pad, out_pad, epilogue, GroupNorm groups)
SEQUENCES = {
    "groupnorm": [(4, 24, 64, 12, 14, 16, 3, 1, 0, 0, W.EPI_RELU_GROUPNORM, 8),
                  (2, 24, 64, 7, 9, 11, 3, 1, 0, 0, W.EPI_RELU_GROUPNORM, 8)],
    "batchnorm": [(4, 16, 48, 10, 12, 14, 4, 2, 1, 0, W.EPI_SCALE_BN_TRAIN_AVGPOOL, 1),
                  (3, 16, 48, 6, 7, 9, 4, 2, 1, 0, W.EPI_SCALE_BN_TRAIN_AVGPOOL, 1)],
    "softmax": [(2, 16, 64, 8, 10, 12, 3, 2, 1, 1, W.EPI_SOFTMAX_SIGMOID, 1),
                (1, 16, 64, 5, 6, 7, 3, 2, 1, 1, W.EPI_SOFTMAX_SIGMOID, 1)],
}


def workload(i, spec):
    n, cin, cout, d, h, w, k, s, p, op, epi, groups = spec
    return W.Workload(f"noalloc{i}", n, cin, cout, d, h, w, k=k, stride=s, pad=p, out_pad=op, bias=True, epi=epi,
                      groups=groups, scale=2.0, seed=31000 + i)


@pytest.mark.gpu
@pytest.mark.parametrize("name", sorted(SEQUENCES))
def test_noalloc_matches_fused_with_workspace(name):
    import torch
    from activation_epilogues_amd import convt3d as C
    for i, spec in enumerate(SEQUENCES[name]):
        wl = workload(i, spec)
        say(f"[case] noalloc {name} call {i}: x {wl.x_shape} cout {wl.cout} k {wl.k} s {wl.stride} "
            f"epi {W.EPI_NAMES[wl.epi]}")
        inp = W.make_inputs(wl)
        g = geom_of(wl)
        call = C.FusedCall(g, wl.epi, wl.groups, wl.eps, wl.scale, want_stats=True)
        assert call.ws_bytes <= C.NOALLOC_SCRATCH_BYTES
        x, w, b = to_dev(inp.x), to_dev(inp.w), to_dev(inp.b)
        gamma, beta = to_dev(inp.gamma), to_dev(inp.beta)
        call.prepack(w)
        call.out.fill_(float("nan"))
        call.workspace.fill_(float("nan"))
        if call.stats is not None:
            call.stats.fill_(float("nan"))
        torch.cuda.synchronize()
        out_ws = call(x, b, gamma, beta).clone()
        stats_ws = None if call.stats is None else call.stats.clone()
        # the same call without a workspace, into fresh NaN-filled outputs
        out_na = torch.full_like(call.out, float("nan"))
        stats_na = None if call.stats is None else torch.full_like(call.stats, float("nan"))
        epi = C.make_epilogue(wl.epi, wl.groups, wl.eps, wl.scale, gamma, beta, stats_na, wl.momentum)
        C.convt3d_fused_noalloc(x, call.w_packed, b, g, epi, out_na)
        torch.cuda.synchronize()
        assert torch.equal(out_na, out_ws), float((out_na - out_ws).abs().max())
        if stats_ws is not None:
            assert torch.equal(stats_na, stats_ws)
        ref = oracle.run_workload(wl, inp)
        out = out_na.cpu().numpy()
        err = max_err(out, ref.out.reshape(out.shape))
        assert err <= TOL, f"max|err| {err:.3e}"
        if stats_na is not None:
            st = stats_na.cpu().numpy()
            np.testing.assert_allclose(st, ref.stats.reshape(st.shape), rtol=1e-5, atol=1e-6)


def test_noalloc_rejects_a_plan_past_the_scratch():
    """A plan needing more workspace than the static scratch is refused on the
    host, before any device work (the pointers are never touched)."""
    from activation_epilogues_amd import convt3d as C
    wl = W.BY_NAME["k4s2_gn"].with_(n=32)
    g = geom_of(wl)
    e = C.make_epilogue(wl.epi, wl.groups)
    assert C.convt3d_workspace_size(g, e) > C.NOALLOC_SCRATCH_BYTES
    fake = 1 << 20  # aligned, never dereferenced
    st = C.convt3d_fused_noalloc(fake, fake, None, g, e, fake, stream=0, check=False)
    assert st == 10, C.status_string(st)
