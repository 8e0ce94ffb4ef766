"""GPU parity of split-KV (fa_fwd_splitkv through the C ABI) against the fp64 oracle.

Splitting the keys of each query tile into runs that are reduced separately and merged by the
rescaling identity must give the same attention ("transformer math: flash attention math",
aicassindra.com, "Proof of exactness": block grouping and order never enter the result), so the
oracle and the tolerances are those of the forward parity tests. Cases: every workload at 3
splits; tails, both head dims, both dtypes, causal or not, with split counts up to more splits
than key tiles (empty splits); a thin grid (B=1, H=2, N=16384) at the heuristic's split count,
also against plain fa_fwd; a reused workspace.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import core
from _compare import check_lse, check_o

pytestmark = pytest.mark.gpu


def _run(q, k, v, causal, scale, num_splits, workspace=None):
    import exact_tiled_softmax_fa_amd as fa
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, num_splits=num_splits,
                        workspace=workspace)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def _compare(o_gpu, lse_gpu, q, k, v, causal, scale, dtype, rows=None):
    B, H, N, d = q.shape
    o_ref, lse_ref = core.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale, causal, rows)
    if rows is not None:
        BH = B * H
        o_gpu = np.stack([o_gpu.reshape(BH, N, d)[i, rows[i]] for i in range(BH)])
        lse_gpu = np.stack([lse_gpu.reshape(BH, N)[i, rows[i]] for i in range(BH)])
    ok_o, rep = check_o(o_gpu, o_ref, dtype)
    ok_l, err_l = check_lse(lse_gpu, lse_ref)
    print(f"[split] O max-abs {rep['max_abs']:.3e} (over tol {rep['n_over_tol']}), lse {err_l:.3e}", flush=True)
    assert ok_o, rep
    assert ok_l, err_l


@pytest.mark.parametrize("name", [w.name for w in workloads.WORKLOADS])
def test_splitkv_workload_parity(name):
    w = workloads.BY_NAME[name]
    print(f"\n[split] {w.name} num_splits=3", flush=True)
    q, k, v = workloads.make_inputs(w)
    o, lse = _run(q, k, v, w.causal, w.scale, 3)
    _compare(o, lse, q, k, v, w.causal, w.scale, w.dtype, workloads.sample_rows(w))
    assert np.isfinite(o).all() and np.isfinite(lse).all()


CASES = [(N, d, causal, dt, sp) for (N, sp) in ((1, 2), (100, 8), (256, 3), (1000, 2), (1000, 7), (2047, 5))
         for d in (64, 128) for causal in (False, True) for dt in ("f16", "bf16")]


@pytest.mark.parametrize("N,d,causal,dt,sp", CASES)
def test_splitkv_shapes(N, d, causal, dt, sp):
    q, k, v = workloads.custom_inputs(1, 3, N, d, dt, 500 + N + d)
    scale = float(np.float32(1 / np.sqrt(d)))
    o, lse = _run(q, k, v, causal, scale, sp)
    _compare(o, lse, q, k, v, causal, scale, dt)


def test_splitkv_thin_grid_matches_oracle_and_fa_fwd():
    import exact_tiled_softmax_fa_amd as fa
    B, H, N, d = 1, 2, 16384, 128
    q, k, v = workloads.custom_inputs(B, H, N, d, "f16", 611)
    scale = float(np.float32(1 / np.sqrt(d)))
    sp = fa.splitkv_heuristic(B, H, N, d, False)
    assert sp > 1
    o, lse = _run(q, k, v, False, scale, sp)
    g = torch.Generator().manual_seed(612)
    rows = np.stack([np.sort(torch.randperm(N, generator=g)[:512].numpy()) for _ in range(B * H)])
    _compare(o, lse, q, k, v, False, scale, "f16", rows)
    o1, lse1 = fa.forward(q.cuda(), k.cuda(), v.cuda(), scale=scale)
    assert np.abs(o1.float().cpu().double().numpy() - o).max() <= 2e-3
    assert np.abs(lse1.cpu().double().numpy() - lse).max() <= 1e-4


def test_splitkv_reuses_a_workspace():
    import exact_tiled_softmax_fa_amd as fa
    need = fa.splitkv_workspace_size(2, 4, 3000, 64, 6)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for (B, H, N, sp, seed) in ((2, 4, 3000, 6, 701), (1, 2, 700, 4, 702)):
        q, k, v = workloads.custom_inputs(B, H, N, 64, "bf16", seed)
        o, lse = _run(q, k, v, True, 0.125, sp, workspace=ws)
        _compare(o, lse, q, k, v, True, 0.125, "bf16")


def test_splitkv_rejects_a_small_workspace():
    import exact_tiled_softmax_fa_amd as fa
    q = torch.zeros(1, 1, 512, 64, dtype=torch.float16, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.forward(q, q, q, num_splits=4, workspace=ws)
    assert e.value.status == 10
