"""GPU parity of fa_fwd_splitkv_blocksparse (split-KV under a block mask, optionally with a window
and key lengths) against the block-sparse fp64 oracle, with the block-sparse tests' rules
(tests/test_gpu_blocksparse.py): rows with no allowed key must come back as o = 0 exactly and
lse = -inf. Split counts are chosen so that some runs of a query tile's keys hold no tile the mask
keeps, or no allowed key of some rows.
"""
import numpy as np
import pytest
import torch

import workloads
from test_gpu_blocksparse import _compare, _mask

pytestmark = pytest.mark.gpu


def _run(q, k, v, m, bq, bk, splits, wl=-1, wr=-1, seqlens=None, scale=None, workspace=None):
    import exact_tiled_softmax_fa_amd as fa
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    o, lse = fa.forward_blocksparse(q.cuda(), k.cuda(), v.cuda(), torch.from_numpy(m).cuda(), bq, bk, wl, wr, sl,
                                    scale=scale, num_splits=splits, workspace=workspace)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


@pytest.mark.parametrize("splits", [2, 3, 7])
@pytest.mark.parametrize("bq,bk", [(64, 64), (128, 192), (256, 128)])
@pytest.mark.parametrize("N,d,dt", [(1000, 64, "bf16"), (2047, 128, "f16")])
def test_random_masks(N, d, dt, bq, bk, splits):
    q, k, v = workloads.custom_inputs(1, 2, N, d, dt, 5100 + N + bq + bk)
    scale = float(np.float32(1 / np.sqrt(d)))
    m = _mask(5101 + N + bq * 3 + bk, (-(-N // bq), -(-N // bk)), 0.3)
    o, lse = _run(q, k, v, m, bq, bk, splits, scale=scale)
    _compare(o, lse, q, k, v, m, bq, bk, scale, dt)


@pytest.mark.parametrize("form", ["head", "batch_head"])
def test_per_head_masks(form):
    B, H, N, d, dt, bq, bk = 2, 2, 900, 128, "bf16", 64, 128
    q, k, v = workloads.custom_inputs(B, H, N, d, dt, 5200)
    shape = (H, -(-N // bq), -(-N // bk)) if form == "head" else (B, H, -(-N // bq), -(-N // bk))
    m = _mask(5201 + len(shape), shape, 0.35)
    o, lse = _run(q, k, v, m, bq, bk, 4, scale=float(np.float32(1 / np.sqrt(d))))
    _compare(o, lse, q, k, v, m, bq, bk, float(np.float32(1 / np.sqrt(d))), dt)


@pytest.mark.parametrize("splits", [2, 5])
@pytest.mark.parametrize("wl,wr,seqlens", [(-1, 0, None), (300, 0, None), (-1, -1, [1100, 1]),
                                           (200, 64, [0, 900])])
def test_with_windows_and_key_lengths(wl, wr, seqlens, splits):
    B, N, d, dt, bq, bk = 2, 1100, 64, "f16", 128, 64
    q, k, v = workloads.custom_inputs(B, 1, N, d, dt, 5300 + max(wl, 0))
    m = _mask(5301, (-(-N // bq), -(-N // bk)), 0.5)
    o, lse = _run(q, k, v, m, bq, bk, splits, wl, wr, seqlens, scale=0.125)
    _compare(o, lse, q, k, v, m, bq, bk, 0.125, dt, wl, wr, seqlens)


def test_runs_the_mask_empties():
    # query block r keeps only key block 0 (r even) or only the last key block (r odd): with 4
    # splits, every query tile has runs with no tile to compute; rows 256 .. 383 keep no key
    N, d, dt, bq, bk = 1500, 128, "f16", 128, 64
    q, k, v = workloads.custom_inputs(1, 1, N, d, dt, 5400)
    nq, nk = -(-N // bq), -(-N // bk)
    m = np.zeros((nq, nk), dtype=np.uint8)
    m[0::2, 0] = 1
    m[1::2, nk - 1] = 1
    m[2] = 0
    o, lse = _run(q, k, v, m, bq, bk, 4, scale=0.088)
    _compare(o, lse, q, k, v, m, bq, bk, 0.088, dt)
    assert np.isneginf(lse[0, 0, 256:384]).all()


def test_agrees_with_the_unsplit_blocksparse_forward_and_reuses_a_workspace():
    import exact_tiled_softmax_fa_amd as fa
    B, H, N, d, bq, bk = 2, 3, 3000, 128, 128, 128
    q, k, v = (t.cuda() for t in workloads.custom_inputs(B, H, N, d, "f16", 5500))
    m = torch.from_numpy(_mask(5501, (-(-N // bq), -(-N // bk)), 0.3)).cuda()
    sl = torch.tensor([3000, 1777], dtype=torch.int32, device="cuda")
    o1, l1 = fa.forward_blocksparse(q, k, v, m, bq, bk, -1, -1, sl)
    ws = torch.empty(fa.splitkv_workspace_size(B, H, N, d, 6), dtype=torch.uint8, device="cuda")
    for splits in (6, 3):  # the same workspace twice, the second call with fewer splits
        o2, l2 = fa.forward_blocksparse(q, k, v, m, bq, bk, -1, -1, sl, num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        assert (o1.float() - o2.float()).abs().max().item() <= 2e-3
        empty = torch.isneginf(l1)
        assert torch.equal(empty, torch.isneginf(l2))
        # each split rounds its probabilities (f16) against its own reference maximum, so the two
        # runs' denominators differ by rounding: both are held to the lse gate against the oracle
        assert (l1[~empty] - l2[~empty]).abs().max().item() <= 1e-3


def test_thin_grid_long_sequence_on_sampled_rows():
    # B1 H2 N16384: 128 query tiles for 256 compute units, the shape split-KV is for
    N, d, dt, bq, bk = 16384, 128, "f16", 128, 128
    q, k, v = workloads.custom_inputs(1, 2, N, d, dt, 5600)
    m = _mask(5601, (N // bq, N // bk), 0.25)
    for i in range(N // bq):
        m[i, i] = 1
    o, lse = _run(q, k, v, m, bq, bk, 2, scale=float(np.float32(1 / np.sqrt(d))))
    rows = np.stack([np.unique(np.r_[0, N - 1, np.random.default_rng(5602 + h).choice(N, 200, replace=False)])
                     for h in range(2)])
    _compare(o, lse, q, k, v, m, bq, bk, float(np.float32(1 / np.sqrt(d))), dt, rows=rows)


def test_past_one_work_list():
    # more than 65536 keys: the kernel that builds each run's list in chunks
    N, d, dt, bq, bk = 65536 + 64 * 3 + 29, 64, "bf16", 64, 64
    q, k, v = workloads.custom_inputs(1, 1, N, d, dt, 5700)
    m = _mask(5701, (-(-N // bq), -(-N // bk)), 0.02)
    for i in range(m.shape[0]):
        m[i, i] = 1
    o, lse = _run(q, k, v, m, bq, bk, 3, scale=0.125)
    rows = np.unique(np.r_[0, N - 1, 65535, 65536, np.random.default_rng(5702).choice(N, 60, replace=False)])[None]
    _compare(o, lse, q, k, v, m, bq, bk, 0.125, dt, rows=rows)
