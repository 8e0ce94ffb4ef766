"""GPU properties with closed-form answers, edge sizes and robustness, all through the C ABI.

Closed forms come from the definition of softmax attention ("transformer math:
flash attention math", section "What we must compute..."): uniform logits give
the mean of the allowed values, a single allowed key gives that key's value,
V = 1 gives 1 (softmax rows sum to 1). The wide-logit cases exercise the
no-overflow argument (same page, "Proof of numerical stability") and masking
before the max ("Pitfalls in implementing the recurrence").
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import core
from _compare import check_lse, check_o

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


def fa():
    import exact_tiled_softmax_fa_amd as m
    return m


def gpu(q, k, v, causal=False, scale=None, variant=0):
    o, lse = fa().forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, variant=variant)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def ref(q, k, v, causal, scale):
    return core.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale, causal)


def say(msg):
    print(f"\n[prop] {msg}", flush=True)


@pytest.mark.parametrize("variant", [1])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
# (600 and 1300 give an odd count of query tiles above one, the case where a paired causal
# workgroup takes the middle tile alone)
@pytest.mark.parametrize("N", [1, 2, 3, 4, 63, 64, 65, 127, 128, 129, 255, 256, 257, 600, 1300, 2047])
def test_tail_sweep(N, causal, d, dt, variant):
    say(f"tail N={N} causal={causal} d={d} {dt} variant={variant}")
    q, k, v = workloads.custom_inputs(2, 3, N, d, dt, seed=100 + N)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = gpu(q, k, v, causal, scale, variant)
    o_ref, lse_ref = ref(q, k, v, causal, scale)
    ok, rep = check_o(o, o_ref, dt)
    assert ok, rep
    assert check_lse(lse, lse_ref)[0]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_values_all_one_give_one(dt, causal):
    say(f"V=1 {dt} causal={causal}")
    q, k, _ = workloads.custom_inputs(1, 4, 700, 128, dt, seed=7, sigma_qk=2.0)
    v = torch.ones_like(q)
    o, _ = gpu(q, k, v, causal)
    assert np.max(np.abs(o - 1.0)) <= 1e-3


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_zero_keys_give_mean_of_values(dt, causal):
    say(f"K=0 {dt} causal={causal}")
    q, _, v = workloads.custom_inputs(1, 2, 300, 64, dt, seed=8)
    k = torch.zeros_like(q)
    o, lse = gpu(q, k, v, causal)
    vd = v.double().numpy()
    cnt = np.arange(1, 301) if causal else np.full(300, 300)
    mean = np.cumsum(vd, axis=2) / cnt[None, None, :, None] if causal else np.broadcast_to(vd.mean(2, keepdims=True), vd.shape)
    ok, rep = check_o(o, mean, dt)
    assert ok, rep
    assert np.max(np.abs(lse - np.log(cnt)[None, None, :])) <= 1e-5


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_causal_row_zero_is_first_value(dt):
    say(f"causal row 0 {dt}")
    q, k, v = workloads.custom_inputs(2, 2, 520, 128, dt, seed=9)
    scale = float(np.float32(1 / math.sqrt(128)))
    o, lse = gpu(q, k, v, True, scale)
    assert np.array_equal(o[:, :, 0], v[:, :, 0].double().numpy())
    dot = (q[:, :, 0].double() * k[:, :, 0].double()).sum(-1).numpy()
    assert np.max(np.abs(lse[:, :, 0] - scale * dot)) <= 1e-4


def test_worked_example_four_keys_on_gpu():
    """The printed four-key example embedded at d = 64: one-hot channel 0, scale 1."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example_four_keys.json")))
    say("worked example (four keys) on GPU")
    q = torch.zeros(1, 1, 4, 64)
    q[..., 0] = 1.0
    k = torch.zeros(1, 1, 4, 64)
    k[0, 0, :, 0] = torch.tensor(g["scores"])
    v = torch.zeros(1, 1, 4, 64)
    v[0, 0, :, 0] = torch.tensor(g["values"])
    o, lse = gpu(q.half(), k.half(), v.half(), False, 1.0)
    assert abs(o[0, 0, 0, 0] - g["o"]["value"]) <= max(g["o"]["tol"], 36.88 * 2 ** -11)
    l = math.exp(lse[0, 0, 0] - 5.0)
    assert abs(l - g["l"]["value"]) <= 1e-3


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_huge_logits_both_signs(dt):
    """q = +-20 * 1, k = 1, d = 128: every logit is +-226 (past fp32 exp overflow at 88.7);
    all keys tie, so O = mean(V) exactly in real arithmetic."""
    say(f"logits +-226 {dt}")
    N, d = 300, 128
    sign = torch.ones(1, 2, N, 1)
    sign[:, 1] = -1
    q = (20.0 * sign).expand(1, 2, N, d).contiguous().to(DTYPES[dt])
    k = torch.ones(1, 2, N, d, dtype=DTYPES[dt])
    _, _, v = workloads.custom_inputs(1, 2, N, d, dt, seed=10)
    scale = float(np.float32(1 / math.sqrt(d)))
    for causal in (False, True):
        o, lse = gpu(q, k, v, causal, scale)
        o_ref, lse_ref = ref(q, k, v, causal, scale)
        assert np.isfinite(o).all() and np.isfinite(lse).all()
        ok, rep = check_o(o, o_ref, dt)
        assert ok, rep
        assert check_lse(lse, lse_ref)[0]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_masked_future_keys_with_huge_logits(dt):
    """Causal, logit(i, j) = 4j: inside every diagonal tile the future keys of a row carry
    logits up to 4*63 above its allowed ones. Taking the block max before masking would put
    the reference there and flush every allowed weight to zero (exp(-252) underflows)."""
    say(f"huge masked logits {dt}")
    N, d = 320, 64
    q = torch.zeros(1, 1, N, d)
    q[..., 0] = 1.0
    k = torch.zeros(1, 1, N, d)
    k[0, 0, :, 0] = 4.0 * torch.arange(N, dtype=torch.float32)
    _, _, v = workloads.custom_inputs(1, 1, N, d, dt, seed=11)
    q, k = q.to(DTYPES[dt]), k.to(DTYPES[dt])
    o, lse = gpu(q, k, v, True, 1.0)
    o_ref, lse_ref = ref(q, k, v, True, 1.0)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    ok, rep = check_o(o, o_ref, dt)
    assert ok, rep
    assert check_lse(lse, lse_ref)[0]


def test_shift_by_constant_channel():
    """A constant-1 key channel: shifting that query channel by delta adds delta*scale to
    every logit of the row, leaving O unchanged and moving lse by delta*scale."""
    say("shift invariance on GPU")
    q, k, v = workloads.custom_inputs(1, 2, 384, 64, "f16", seed=12)
    k[..., 63] = 1.0
    q[..., 63] = 0.0
    q2 = q.clone()
    q2[..., 63] = 8.0
    scale = 0.125
    o1, l1 = gpu(q, k, v, False, scale)
    o2, l2 = gpu(q2, k, v, False, scale)
    assert np.max(np.abs(o1 - o2)) <= 2e-3
    assert np.max(np.abs((l2 - l1) - 1.0)) <= 1e-3


def test_repeat_runs_are_bit_identical():
    say("20 repeats bit-identical")
    w = workloads.BY_NAME["B4-H16-N2047-d64-bf16"]
    q, k, v = (t.cuda() for t in workloads.make_inputs(w))
    o0, l0 = fa().forward(q, k, v)
    for _ in range(19):
        o, l = fa().forward(q, k, v)
        assert torch.equal(o, o0) and torch.equal(l, l0)


def test_lse_optional_and_streams():
    say("lse=None and a side stream")
    q, k, v = (t.cuda() for t in workloads.custom_inputs(1, 2, 200, 64, "f16", seed=13))
    o_ref, l_ref = fa().forward(q, k, v)
    o = fa().forward(q, k, v, return_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o2, l2 = fa().forward(q, k, v)
    s.synchronize()
    assert torch.equal(o2, o_ref) and torch.equal(l2, l_ref)


def test_single_hip_runtime_in_process():
    """The library must bind to the HIP runtime torch already loaded (one libamdhip64)."""
    fa().lib()
    maps = open("/proc/self/maps").read()
    paths = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(paths) == 1, paths


@pytest.mark.parametrize("tau", [None, 0.0, 3.0])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_scores_rising_along_the_keys(dt, tau):
    """Logit(i, j) = slope * j + noise: every key tile raises every row's maximum, so the kernel
    moves its reference (and recomputes a tile's exponentials) again and again, at the default
    threshold (None: 8), at 0 (the reference is always the running max) and at 3. The result
    must still be the definition's."""
    say(f"rising logits {dt} tau={tau}")
    B, H, N, d = 1, 2, 1100, 128
    scale = float(np.float32(1 / math.sqrt(d)))
    g = torch.Generator().manual_seed(77)
    # channel 0 carries the slope (q = 1, k_j = slope * j / scale), the others small noise
    slope = 0.05
    q = torch.randn(B, H, N, d, generator=g) * 0.1
    k = torch.randn(B, H, N, d, generator=g) * 0.1
    q[..., 0] = 1.0
    k[..., 0] = torch.arange(N, dtype=torch.float32) * (slope / scale)
    q, k = q.to(DTYPES[dt]), k.to(DTYPES[dt])
    _, _, v = workloads.custom_inputs(B, H, N, d, dt, seed=78)
    o, lse = fa().forward(q.cuda(), k.cuda(), v.cuda(), scale=scale, rescale_threshold_log2=tau)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().double().numpy(), lse.cpu().double().numpy()
    o_ref, lse_ref = ref(q, k, v, False, scale)
    # the scores span about slope * N = 55 natural-log units: far beyond one tile's threshold
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    ok, rep = check_o(o, o_ref, dt)
    assert ok, rep
    ok_l, err_l = check_lse(lse, lse_ref)
    assert ok_l, err_l
