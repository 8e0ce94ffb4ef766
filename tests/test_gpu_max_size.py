"""GPU parity at the largest sizes the library accepts, against the fp64 oracle on sampled rows.

One head of q, k or v may hold up to 2^31 - 1 bytes (the kernels address a head with 32-bit
offsets), so N = 8388607 at d = 128. A sliding window of 256 keys keeps that case to a few
milliseconds of GPU work; the oracle checks each sampled row on the keys its window allows (a
sub-problem of at most 256 keys, the row last). A 262181-key head runs plain and causal attention
in full. Inputs are seeded N(0, 1) draws, made on the GPU at these sizes (the same recipe as
workloads.custom_inputs, with a CUDA generator). Tolerances are the forward's.
"""
import numpy as np
import pytest
import torch

from oracle import core
from _compare import check_lse, check_o

pytestmark = pytest.mark.gpu


def _gpu_inputs(B, H, N, d, dtype, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    dt = torch.float16 if dtype == "f16" else torch.bfloat16
    return [torch.randn(B, H, N, d, generator=g, device="cuda", dtype=torch.float32).to(dt) for _ in range(3)]


def _rows(N, seed, count=12):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 255, 256, N // 2, N - 256, N - 2, N - 1]
    return np.unique(np.r_[fixed, rng.choice(N, count, replace=False)]).astype(np.int64)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_largest_head_with_a_local_window(dt):
    import exact_tiled_softmax_fa_amd as fa
    d = 128
    N = (2**31 - 1) // (d * 2)  # 8388607 rows: one head of q, k or v just under 2 GiB
    wl = 255
    q, k, v = _gpu_inputs(1, 1, N, d, dt, 7100 + len(dt))
    scale = float(np.float32(1 / np.sqrt(d)))
    o, lse = fa.forward_masked(q, k, v, wl, 0, scale=scale)
    torch.cuda.synchronize()
    rows = _rows(N, 7102)
    print(f"[max size] N={N} d={d} {dt} window {wl}/0: checking {len(rows)} rows", flush=True)
    o_ref, lse_ref, o_gpu, lse_gpu = [], [], [], []
    for i in map(int, rows):
        lo = max(0, i - wl)
        sub = [t[:, :, lo:i + 1].double().cpu().numpy() for t in (q, k, v)]
        L = i + 1 - lo
        ro, rl = core.attention_masked(*sub, scale, wl, 0, None, np.array([[L - 1]], dtype=np.int64))
        o_ref.append(ro[0, 0])
        lse_ref.append(rl[0, 0])
        o_gpu.append(o[0, 0, i].float().cpu().double().numpy())
        lse_gpu.append(float(lse[0, 0, i]))
    ok_o, rep = check_o(np.array(o_gpu), np.array(o_ref), dt)
    ok_l, err_l = check_lse(np.array(lse_gpu), np.array(lse_ref))
    print(f"[max size] O max-abs {rep['max_abs']:.3e}, lse {err_l:.3e}", flush=True)
    assert ok_o, rep
    assert ok_l, err_l


@pytest.mark.parametrize("causal", [False, True])
def test_long_head_in_full(causal):
    import exact_tiled_softmax_fa_amd as fa
    N, d, dt = 262144 + 37, 64, "bf16"
    q, k, v = _gpu_inputs(1, 1, N, d, dt, 7200 + int(causal))
    scale = float(np.float32(1 / np.sqrt(d)))
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rows = _rows(N, 7201, 6)
    qd, kd, vd = (t.double().cpu().numpy() for t in (q, k, v))
    o_ref, lse_ref = core.attention(qd, kd, vd, scale, causal, rows[None, :])
    o_gpu = o[0, 0, torch.from_numpy(rows).cuda()].float().cpu().double().numpy()[None]
    lse_gpu = lse[0, 0, torch.from_numpy(rows).cuda()].cpu().double().numpy()[None]
    ok_o, rep = check_o(o_gpu, o_ref, dt)
    ok_l, err_l = check_lse(lse_gpu, lse_ref)
    print(f"[long] N={N} causal={causal}: O max-abs {rep['max_abs']:.3e}, lse {err_l:.3e}", flush=True)
    assert ok_o, rep
    assert ok_l, err_l
