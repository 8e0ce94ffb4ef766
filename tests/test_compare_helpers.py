"""The comparison helpers the GPU tests rely on, pinned on the CPU."""
import numpy as np

from _compare import check_lse, check_o, ulp


def test_ulp_values():
    assert ulp(1.0, "f16") == 2.0 ** -10 and ulp(1.5, "f16") == 2.0 ** -10 and ulp(2.0, "f16") == 2.0 ** -9
    assert ulp(3.0, "bf16") == 2.0 ** -6 and ulp(-0.75, "bf16") == 2.0 ** -8
    # subnormal range and zero take the subnormal spacing
    assert ulp(1e-6, "f16") == 2.0 ** -24 and ulp(0.0, "f16") == 2.0 ** -24 and ulp(0.0, "bf16") == 2.0 ** -133


def test_check_o_allows_only_rounding_beyond_tol():
    ref = np.array([0.1, 5.0, -3.0])
    ok, rep = check_o(ref + np.array([1.9e-3, 0.0, 0.0]), ref, "f16")
    assert ok and rep["n_over_tol"] == 0
    # beyond tol but within tol + ulp/2 at |ref| >= 2: allowed and counted
    ok, rep = check_o(ref + np.array([0.0, 2e-3 + 0.4 * 2.0 ** -8, 0.0]), ref, "f16")
    assert ok and rep["n_over_tol"] == 1
    ok, _ = check_o(ref + np.array([2.1e-3, 0.0, 0.0]), ref, "f16")
    assert not ok
    ok, _ = check_o(np.array([np.nan, 5.0, -3.0]), ref, "f16")
    assert not ok


def test_check_lse():
    assert check_lse([1.0, 2.0], [1.0009, 2.0])[0]
    assert not check_lse([1.0, 2.0], [1.0011, 2.0])[0]
