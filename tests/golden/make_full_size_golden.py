"""Write the expected values of the full-size workloads, computed by the fp64
CPU oracle only (nothing here touches the GPU path):

    python tests/golden/make_full_size_golden.py [name ...]

For each workload it stores, in tests/golden/full_<name>.npz:
  * checksums of the seeded float32 inputs (so a changed input stream is caught),
  * the raw transposed-convolution output at sampled voxels,
  * the final output at the same sampled voxels (GroupNorm / softmax) or the
    whole pooled [n, cout] output (BatchNorm + average pool),
  * the statistics the library can export: GroupNorm [n, groups, 2] =
    (mean, rstd), BatchNorm [cout, 2] = (batch mean, biased variance).
Sample voxels are drawn with numpy default_rng(7) over the whole output, plus
the eight corners of every sample/channel pair's first and last channel.
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from activation_epilogues_amd import workloads as W  # noqa: E402

N_SAMPLES = 4096


def checksums(inp):
    out = {}
    for k in ("x", "w", "b", "gamma", "beta"):
        a = getattr(inp, k)
        if a is not None:
            out["sum_" + k] = np.float64(a.astype(np.float64).sum())
            out["head_" + k] = a.reshape(-1)[:8].copy()
    return out


def sample_index(shape, rng):
    N, C, D, H, Wd = shape
    idx = np.stack([rng.integers(0, s, N_SAMPLES) for s in shape], axis=1)
    corners = []
    for n in (0, N - 1):
        for c in (0, C - 1):
            for d in (0, D - 1):
                for h in (0, H - 1):
                    for w in (0, Wd - 1):
                        corners.append((n, c, d, h, w))
    return np.concatenate([idx, np.array(corners)], axis=0).astype(np.int64)


def make(name):
    wl = W.BY_NAME[name]
    inp = W.make_inputs(wl)
    t0 = time.time()
    res = oracle.run_workload(wl, inp)
    dt = time.time() - t0
    data = checksums(inp)
    rng = np.random.default_rng(7)
    idx = sample_index(res.y.shape, rng)
    data["sample_index"] = idx
    data["raw_at_samples"] = res.y[tuple(idx.T)]
    if wl.epi == W.EPI_SCALE_BN_TRAIN_AVGPOOL:
        data["out"] = res.out
    else:
        data["out_at_samples"] = res.out[tuple(idx.T)]
    if res.stats is not None:
        data["stats"] = res.stats
    data["oracle_seconds"] = np.float64(dt)
    path = os.path.join(HERE, f"full_{name}.npz")
    np.savez_compressed(path, **data)
    print(f"{name}: oracle {dt:.1f} s, wrote {path}", flush=True)


if __name__ == "__main__":
    names = sys.argv[1:] or [wl.name for wl in W.WORKLOADS if wl.name != "tiny_gn"]
    for nm in names:
        make(nm)
