"""GPU parity of fa_fwd_splitkv_masked (split-KV under a sliding window and key lengths) against
the masked fp64 oracle, with the masked tests' rules (tests/test_gpu_masked.py): rows with no
allowed key must come back as o = 0 exactly and lse = -inf. Split counts are chosen so that some
splits of a query tile's window hold no allowed key of some rows, or no tile at all.
"""
import numpy as np
import pytest
import torch

import workloads
from test_gpu_masked import _compare

pytestmark = pytest.mark.gpu


def _run(q, k, v, wl, wr, seqlens, scale, splits, workspace=None):
    import exact_tiled_softmax_fa_amd as fa
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    o, lse = fa.forward_masked(q.cuda(), k.cuda(), v.cuda(), wl, wr, sl, scale=scale, num_splits=splits,
                               workspace=workspace)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


@pytest.mark.parametrize("splits", [2, 3, 7])
@pytest.mark.parametrize("wl,wr", [(0, 0), (100, 0), (257, 0), (63, 63), (-1, 5), (200, -1), (1, 300)])
@pytest.mark.parametrize("N,d,dt", [(1000, 128, "bf16"), (700, 64, "f16")])
def test_sliding_windows(wl, wr, N, d, dt, splits):
    q, k, v = workloads.custom_inputs(1, 2, N, d, dt, 3100 + N + max(wl, 0))
    scale = float(np.float32(1 / np.sqrt(d)))
    o, lse = _run(q, k, v, wl, wr, None, scale, splits)
    _compare(o, lse, q, k, v, wl, wr, None, scale, dt)


@pytest.mark.parametrize("splits", [2, 5])
@pytest.mark.parametrize("wl,wr,seqlens", [(-1, -1, [700, 513, 1]), (-1, 0, [64, 700, 300]),
                                           (128, 0, [0, 650, 699]), (50, 10, [700, 0, 256])])
@pytest.mark.parametrize("d,dt", [(64, "bf16"), (128, "f16")])
def test_key_padding(wl, wr, seqlens, d, dt, splits):
    q, k, v = workloads.custom_inputs(3, 2, 700, d, dt, 3200 + d)
    scale = float(np.float32(1 / np.sqrt(d)))
    o, lse = _run(q, k, v, wl, wr, seqlens, scale, splits)
    _compare(o, lse, q, k, v, wl, wr, seqlens, scale, dt)


def test_agrees_with_the_unsplit_masked_forward_and_reuses_a_workspace():
    import exact_tiled_softmax_fa_amd as fa
    q, k, v = (t.cuda() for t in workloads.custom_inputs(2, 3, 3000, 128, "f16", 3300))
    sl = torch.tensor([3000, 1777], dtype=torch.int32, device="cuda")
    o1, l1 = fa.forward_masked(q, k, v, 1023, 0, sl)
    ws = torch.empty(fa.splitkv_workspace_size(2, 3, 3000, 128, 4), dtype=torch.uint8, device="cuda")
    for splits in (4, 3):  # the same workspace twice, the second call with fewer splits
        o2, l2 = fa.forward_masked(q, k, v, 1023, 0, sl, num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        assert (o1.float() - o2.float()).abs().max().item() <= 2e-3
        empty = torch.isneginf(l1)  # rows past the second batch's keys and window keep no key
        assert empty.any() and torch.equal(empty, torch.isneginf(l2))
        assert (l1[~empty] - l2[~empty]).abs().max().item() <= 1e-4


def test_window_on_a_thin_grid():
    """The case split-KV is for: few query tiles (B1 H2 N16384) and a long window."""
    w = workloads.BY_NAME["B1-H2-N16384-d128-f16"]
    q, k, v = workloads.make_inputs(w)
    o, lse = _run(q, k, v, 4095, 0, None, w.scale, 4)
    _compare(o, lse, q, k, v, 4095, 0, None, w.scale, w.dtype, rows=workloads.sample_rows(w))
