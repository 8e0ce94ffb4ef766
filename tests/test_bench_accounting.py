"""bench.py's flop accounting for the masked and block-sparse lines (no GPU): the allowed-pair
counts it prices the GPU run and the CPU oracle baseline by, against brute force."""
import numpy as np
import pytest

import bench
import workloads


@pytest.mark.parametrize("N,window", [(300, (31, 0)), (300, (-1, 5)), (257, (0, 0)), (100, (200, -1)), (64, (-1, -1))])
def test_window_keys(N, window):
    wl, wr = window
    want = [sum(1 for j in range(N) if (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr)) for i in range(N)]
    np.testing.assert_array_equal(bench._window_keys(np.arange(N), N, window), want)


@pytest.mark.parametrize("N,bs,p", [(300, 64, 0.5), (256, 128, 0.3), (1000, 192, 0.6)])
def test_block_mask_pairs(N, bs, p):
    w = workloads.Workload("t", 1, 1, N, 64, "f16", False, 1.0, 7, None)
    m = workloads.make_block_mask(w, bs, p)
    assert m.shape == (-(-N // bs),) * 2 and np.all(np.diag(m) == 1)
    want = sum(int(m[i // bs, j // bs]) for i in range(N) for j in range(N))
    assert workloads.block_mask_pairs(m, N, bs, bs) == want


def test_baselines_run_the_matching_oracle():
    w = workloads.BY_NAME["B1-H1-N256-d64-f16"]
    assert "masked oracle, window 31/0" in bench.cpu_baseline(w, window=(31, 0))["sample"]
    m = workloads.make_block_mask(w, 64, 0.5)
    assert "block-sparse oracle" in bench.cpu_baseline(w, blocks=(64, m))["sample"]
    assert "window 31/0" in bench.cpu_baseline_bwd(w, window=(31, 0))["sample"]
    assert "64x64 block mask" in bench.cpu_baseline_bwd(w, blocks=(64, m))["sample"]
    assert "three-pass" in bench.cpu_baseline(w)["sample"]
