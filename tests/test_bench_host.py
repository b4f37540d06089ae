"""Host-side checks of bench.py's work counts (no GPU): the flop and pair
counts the roofline divides by agree with counts taken from the oracle's mask."""
import numpy as np
import pytest

import bench
from oracle import attention as A


@pytest.mark.parametrize("Nq,Nk,q0,k0", [(1, 1, 0, 0), (37, 37, 0, 0), (20, 50, 100, 70), (50, 20, 10, 40),
                                         (16, 16, 0, 100), (64, 128, 200, 0)])
def test_causal_pairs_match_mask(Nq, Nk, q0, k0):
    m = A.visible(q0 + np.arange(Nq), k0 + np.arange(Nk))
    assert bench.causal_pairs(Nq, Nk, q0, k0) == int(m.sum())


@pytest.mark.parametrize("N,W,S", [(1, 1, 0), (50, 7, 0), (50, 7, 4), (300, 64, 4), (100, 200, 4), (4096, 4096, 4)])
def test_window_pairs_match_oracle(N, W, S):
    assert bench.window_pairs(N, W, S) == A.visible_pairs(N, W, S)


def test_flops_of_the_32k_workload():
    # 4 D flops per kept pair per query head: 4 * 128 * 32 * N (N + 1) / 2 at N = 32768
    assert bench.prefill_flops(1, 32, 32768, 32768, 128) == 4.0 * 128 * 32 * 32768 * 32769 / 2


def test_more_than_one_gpu_is_refused():
    """The benchmark runs on one GPU: --gpus above 1 exits with status 2 and a
    message, before anything touches a device."""
    import json
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "8"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]
