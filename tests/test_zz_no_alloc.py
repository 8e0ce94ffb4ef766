"""fa_fwd_splitkv_noalloc (include/fa_fwd.h) through the C ABI: the split-KV forward with its partial
results in the library's fixed device scratch instead of a caller workspace.

It runs the kernels of fa_fwd_splitkv, so its outputs must equal that entry point's (with a workspace
the caller allocates) bit for bit, and both must match the fp64 oracle under the forward tolerances.
Two calls in a row, the second on a smaller problem, so the second reuses the scratch the first left.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import core
from _compare import check_lse, check_o

pytestmark = pytest.mark.gpu

# (B, H, N, d, dtype, causal, splits); the second call is the smaller one
CALLS = [(1, 2, 4000, 128, "f16", False, 3), (1, 1, 700, 64, "bf16", True, 2)]


def _noalloc(q, k, v, causal, scale, splits):
    import exact_tiled_softmax_fa_amd as fa
    B, H, N, d = q.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream().cuda_stream
    st = fa.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H,
                                   N, d, scale, causal, stream, 1 if q.dtype == torch.bfloat16 else 0, splits)
    torch.cuda.synchronize()
    assert st == 0, fa.status_string(st)
    return o, lse


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    import exact_tiled_softmax_fa_amd as fa
    for i, (B, H, N, d, dt, causal, splits) in enumerate(CALLS):
        print(f"\n[noalloc] call {i}: B{B} H{H} N{N} d{d} {dt} causal={causal} splits={splits}", flush=True)
        q, k, v = workloads.custom_inputs(B, H, N, d, dt, 7100 + i)
        scale = float(np.float32(1 / np.sqrt(d)))
        qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
        o1, l1 = _noalloc(qc, kc, vc, causal, scale, splits)
        o2, l2 = fa.forward(qc, kc, vc, causal=causal, scale=scale, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), "outputs differ from fa_fwd_splitkv's"
        assert torch.equal(l1, l2), "lse differs from fa_fwd_splitkv's"
        o_ref, lse_ref = core.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale, causal)
        ok_o, rep = check_o(o1.float().cpu().double().numpy(), o_ref, dt)
        ok_l, err_l = check_lse(l1.cpu().double().numpy(), lse_ref)
        print(f"[noalloc] call {i}: O max-abs {rep['max_abs']:.3e}, lse max-abs {err_l:.3e}", flush=True)
        assert ok_o, rep
        assert ok_l, err_l


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    import exact_tiled_softmax_fa_amd as fa
    q = torch.zeros(1, 8, 8192, 128, dtype=torch.float16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(1, 8, 8192, dtype=torch.float32, device="cuda")
    st = fa.fa_fwd_splitkv_noalloc(q.data_ptr(), q.data_ptr(), q.data_ptr(), o.data_ptr(), lse.data_ptr(), 1, 8, 8192,
                                   128, 0.088, 0, torch.cuda.current_stream().cuda_stream, 0, 2)
    assert st == 11, fa.status_string(st)
