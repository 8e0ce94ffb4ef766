"""The host-CPU variant (fa_fwd_cpu, include/fa_cpu.h) against the fp64 oracle. Runs without a GPU.

Same tolerances as the GPU forward (it computes in fp32 throughout, so it sits well inside them);
tails around the 32-row query tiles and 64-key blocks, both head dims, both dtypes, causal or not;
the result must not depend on the thread count; wide logits must not overflow. The shape cases run
under every instruction-set build the test machine has (AVX-512, AVX2, plain C++; FA_CPU_ISA
selects a lower one than the best).
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import core
from _compare import check_lse, check_o


def _cpu_flags():
    try:
        return open("/proc/cpuinfo").read()
    except OSError:
        return ""


ISAS = ["generic"] + (["avx2"] if " avx2" in _cpu_flags() else []) + (["best"] if " avx512f" in _cpu_flags() else [])


@pytest.fixture(params=ISAS)
def isa(request, monkeypatch):
    if request.param != "best":
        monkeypatch.setenv("FA_CPU_ISA", request.param)
    return request.param


def _check(q, k, v, causal, scale, dtype, threads=0):
    import exact_tiled_softmax_fa_amd as fa
    o, lse = fa.forward_cpu(q, k, v, causal=causal, scale=scale, num_threads=threads)
    o_ref, lse_ref = core.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale, causal)
    ok_o, rep = check_o(o.float().double().numpy(), o_ref, dtype)
    ok_l, err_l = check_lse(lse.double().numpy(), lse_ref)
    assert ok_o, rep
    assert ok_l, err_l
    return o, lse, rep, err_l


@pytest.mark.parametrize("N", [1, 31, 32, 33, 64, 65, 200])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_cpu_tiled_matches_oracle(N, d, causal, dt, isa):
    q, k, v = workloads.custom_inputs(2, 2, N, d, dt, 1000 + N + d)
    _check(q, k, v, causal, float(np.float32(1 / np.sqrt(d))), dt, threads=3)


def test_cpu_tiled_first_workload_all_rows():
    w = workloads.BY_NAME["B1-H1-N256-d64-f16"]
    q, k, v = workloads.make_inputs(w)
    _, _, rep, err_l = _check(q, k, v, w.causal, w.scale, w.dtype)
    assert rep["max_abs"] < 5e-4 and err_l < 1e-5  # fp32 throughout: well inside the tolerance


def test_cpu_tiled_wide_logits(isa):
    q, k, v = workloads.custom_inputs(1, 2, 300, 128, "bf16", 1100, sigma_qk=4.0)
    _check(q, k, v, True, float(np.float32(1 / np.sqrt(128))), "bf16")


def test_cpu_tiled_is_independent_of_the_thread_count(isa):
    import exact_tiled_softmax_fa_amd as fa
    q, k, v = workloads.custom_inputs(2, 3, 333, 64, "f16", 1200)
    a = fa.forward_cpu(q, k, v, causal=True, num_threads=1)
    for t in (2, 5, 0):
        b = fa.forward_cpu(q, k, v, causal=True, num_threads=t)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_cpu_tiled_rejects_bad_arguments():
    import exact_tiled_softmax_fa_amd as fa
    z = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.forward_cpu(z, z, z.float())
    assert fa.fa_fwd_cpu(None, z.data_ptr(), z.data_ptr(), z.data_ptr(), None, 1, 1, 8, 64, 0.1, 0, 0, 1) == 1
    o = torch.empty_like(z)
    assert fa.fa_fwd_cpu(z.data_ptr(), z.data_ptr(), z.data_ptr(), o.data_ptr(), None, 1, 1, 8, 96, 0.1, 0, 0, 1) == 3
    assert fa.fa_fwd_cpu(z.data_ptr(), z.data_ptr(), z.data_ptr(), z.data_ptr(), None, 1, 1, 8, 64, 0.1, 0, 0, 1) == 8  # FA_ERR_ALIAS
    assert fa.fa_fwd_cpu(z.data_ptr(), z.data_ptr(), z.data_ptr(), o.data_ptr(), None, 1, 1, 8, 64, -1.0, 0, 0, 1) == 6


def test_cpu_tiled_builds_agree():
    """The three builds compute the same recurrence in fp32; only the summation order differs."""
    import os
    import exact_tiled_softmax_fa_amd as fa
    q, k, v = workloads.custom_inputs(1, 2, 500, 128, "bf16", 1300)
    outs = {}
    for name in ISAS:
        if name == "best":
            os.environ.pop("FA_CPU_ISA", None)
        else:
            os.environ["FA_CPU_ISA"] = name
        try:
            outs[name] = fa.forward_cpu(q, k, v, causal=True)
        finally:
            os.environ.pop("FA_CPU_ISA", None)
    ref = outs["generic"]
    for name, (o, lse) in outs.items():
        assert (o.float() - ref[0].float()).abs().max().item() <= 2 ** -7  # one bf16 ulp at |o| < 1
        assert (lse - ref[1]).abs().max().item() <= 1e-5
