"""bench.py on the host: the one-GPU contract and the figures it derives
without a GPU (step statistics, the effective-FLOP counts)."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synthetic as S  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_step_stats():
    st = bench.step_stats([3.0, 1.0, 2.0, 10.0, 4.0])
    assert st["median"] == 3.0 and st["min"] == 1.0
    assert st["p90"] == float(np.percentile([1, 2, 3, 4, 10], 90))


def test_effective_flops_of_the_workloads():
    # 720p at 25 % keep: 4 * B * H * D * 122,880 queries * 480 * 64 keys
    wl = S.WORKLOADS["prism720p"]
    assert wl.effective_flops() == 4.0 * 2 * 24 * 128 * 122880 * 480 * 64
    # the ragged clip counts whole tiles, as the kernels compute them
    assert S.WORKLOADS["prism720p_ragged"].effective_flops() == wl.effective_flops()
    # one keep count for every head reproduces the fixed-keep count
    assert bench.varkeep_flops(wl, [480] * wl.heads) == wl.effective_flops()
