"""The seeded input generator: deterministic, right shapes and dtypes, valid row samples."""
import numpy as np
import torch

import workloads


def test_inputs_are_deterministic_and_shaped():
    w = workloads.WORKLOADS[0]
    a = workloads.make_inputs(w)
    b = workloads.make_inputs(w)
    for x, y in zip(a, b):
        assert x.shape == (w.B, w.H, w.N, w.d)
        assert x.dtype == torch.float16
        assert torch.equal(x, y)
    # q, k, v are different draws
    assert not torch.equal(a[0], a[1])


def test_wide_logit_workload_scales_q_and_k_only():
    w = workloads.BY_NAME["B1-H8-N32768-d128-bf16-causal-qk4"]
    small = workloads.Workload("t", 1, 1, 4096, 128, "bf16", True, 4.0, w.seed, None)
    q, k, v = workloads.make_inputs(small)
    assert 3.5 < q.float().std().item() < 4.5
    assert 3.5 < k.float().std().item() < 4.5
    assert 0.9 < v.float().std().item() < 1.1


def test_row_samples():
    for w in workloads.WORKLOADS:
        rows = workloads.sample_rows(w)
        if w.rows_per_head is None:
            assert rows is None
            continue
        assert rows.shape == (w.B * w.H, w.rows_per_head)
        for r in rows:
            assert len(np.unique(r)) == len(r)
            assert r[0] == 0 and r[-1] == w.N - 1
            assert np.all(np.diff(r) > 0)


def test_scale_is_fp32_inverse_sqrt():
    for w in workloads.WORKLOADS:
        assert w.scale == float(np.float32(1 / np.sqrt(w.d)))
    assert workloads.BY_NAME["B1-H1-N256-d64-f16"].scale == 0.125
