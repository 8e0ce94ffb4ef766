"""A CPU model of the backward kernels' designed roundings, run on every shape of
tests/test_gpu_backward_edges.py, pins that test's elementwise bound independently of the GPU.

The model follows the arithmetic the kernels are built to do ("Decoding flash attention",
bibekananda.in, "The backward pass": recompute p from the saved statistic, then the chain rule
through softmax), with each rounding placed where the kernels place it:
  forward  p = exp(s - m) in fp32, rounded to the input dtype as the second product's operand;
           O = (sum_j p~_j v_j) / l in fp32, stored rounded to the dtype, and lse = m + ln l in
           fp32, with l the sum of the rounded p in f16 and of the unrounded p in bf16;
  backward D_i = dO_i . O_i from the stored O (fp32 sum); p_ij = exp(s_ij - lse_i) in fp32;
           dP = dO V^T and dS = p (dP - D) in fp32; dV = p~^T dO, dK = scale dS~^T Q and
           dQ = scale dS~ K with p~, dS~ rounded to the dtype as operands, fp32 sums; each
           gradient stored rounded to the dtype.
Sums are formed in fp64 and rounded to fp32 once (the kernels' fp32 accumulation order differs,
well below the dtype roundings). Every error the model makes against the fp64 oracle must be at
most half of the GPU test's bound (its 2x allowance for accumulation order and the exponential's
approximation is thus not consumed by the designed roundings alone), so the bound is not fitted to
GPU results. The check is on the value before the gradient's own rounding to the dtype: that last
rounding is the half ulp the bound adds on its own, and on gradients in the f16 subnormal range
(a few 1e-8) it is nearly all of the bound. Runs without a GPU.
"""
import numpy as np
import pytest

import workloads
from oracle import core
from _compare import ulp
from test_gpu_backward_edges import CASES, _allowed, _bounds


def _round(x, dt):
    x = np.asarray(x, dtype=np.float32)
    if dt == "f16":
        return x.astype(np.float16).astype(np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def model_backward(q, k, v, dout, scale, wl, wr, seqlens, dt, stored=True):
    """(dq, dk, dv) as fp64 arrays [G, N, d]: the model's stored values, or with stored=False the fp32
    values just before their rounding to the dtype."""
    B, H, N, d = q.shape
    outs = []
    for g in range(B * H):
        Q, K, V, dO = (x.reshape(B * H, N, d)[g].double().numpy() for x in (q, k, v, dout))
        allowed = _allowed(N, g // H, wl, wr, seqlens)
        s = np.where(allowed, _f32(scale * _f32(Q @ K.T)), -np.inf).astype(np.float32)
        # forward
        m = s.max(axis=1, keepdims=True)
        m = np.where(np.isfinite(m), m, np.float32(0))
        p = _f32(np.exp(s.astype(np.float64) - m))
        pt = _round(p, dt)
        summed = p if dt == "bf16" else pt
        l = _f32(summed.astype(np.float64).sum(axis=1, keepdims=True))
        o = _round(_f32(_f32(pt.astype(np.float64) @ V) / np.where(l > 0, l, 1)), dt)
        lse = np.where(l > 0, _f32(m + np.log(np.where(l > 0, l, 1).astype(np.float64))), -np.inf)
        # backward
        D = _f32((dO * o.astype(np.float64)).sum(axis=1, keepdims=True))
        with np.errstate(invalid="ignore"):  # rows with no allowed key: lse = -inf, p = 0
            pb = np.where(allowed & np.isfinite(lse), _f32(np.exp(s.astype(np.float64) - lse)), np.float32(0))
        dP = _f32(dO @ V.T)
        dS = _f32(pb.astype(np.float64) * (dP.astype(np.float64) - D))
        dSt = _round(dS, dt).astype(np.float64)
        out = (lambda x: _round(x, dt)) if stored else (lambda x: x)
        dv = out(_f32(_round(pb, dt).astype(np.float64).T @ dO))
        dk = out(_f32(scale * _f32(dSt.T @ Q)))
        dq = out(_f32(scale * _f32(dSt @ K)))
        outs.append((dq, dk, dv))
    return [np.stack([o[i] for o in outs]).astype(np.float64) for i in range(3)]


@pytest.mark.parametrize("B,H,N,d,dt,sigma,wl,wr,seqlens", CASES)
def test_designed_roundings_use_at_most_half_the_bound(B, H, N, d, dt, sigma, wl, wr, seqlens):
    q, k, v = workloads.custom_inputs(B, H, N, d, dt, 8000 + N + d, sigma_qk=sigma)
    dout = workloads.custom_inputs(B, H, N, d, dt, 8001 + N + d)[0]
    scale = float(np.float32(1 / np.sqrt(d)))
    refs = core.attention_backward_masked(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                          dout.double().numpy(), scale, wl, wr, seqlens)[:3]
    pre = model_backward(q, k, v, dout, scale, wl, wr, seqlens, dt, stored=False)
    stored = model_backward(q, k, v, dout, scale, wl, wr, seqlens, dt)
    bounds = _bounds(q, k, v, dout, scale, wl, wr, seqlens, dt)
    G = B * H
    for name, x, st, r, bnd in zip(("dq", "dk", "dv"), pre, stored, refs, bounds):
        ref = np.asarray(r).reshape(G, N, d)
        worst = float((np.abs(x - ref) / (bnd + 1e-30)).max())
        assert np.all(np.abs(x - ref) <= 0.5 * bnd + 1e-30), f"{name}: designed roundings reach {worst:.3f} of the bound"
        # and the stored value within the GPU test's limit
        assert np.all(np.abs(st - ref) <= bnd + 0.5 * ulp(ref, dt) + 1e-30), name


def test_the_model_sees_what_the_bound_is_for():
    """The model is not trivially exact: on the peaked f16 case its dq error is a visible fraction of
    the bound (a model with a rounding left out would show far less)."""
    B, H, N, d, dt, sigma, wl, wr, seqlens = CASES[0]
    q, k, v = workloads.custom_inputs(B, H, N, d, dt, 8000 + N + d, sigma_qk=sigma)
    dout = workloads.custom_inputs(B, H, N, d, dt, 8001 + N + d)[0]
    scale = float(np.float32(1 / np.sqrt(d)))
    refs = core.attention_backward_masked(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                          dout.double().numpy(), scale, wl, wr, seqlens)[:3]
    dq = model_backward(q, k, v, dout, scale, wl, wr, seqlens, dt, stored=False)[0]
    bq = _bounds(q, k, v, dout, scale, wl, wr, seqlens, dt)[0]
    ref = np.asarray(refs[0]).reshape(dq.shape)
    frac = float((np.abs(dq - ref) / (bq + 1e-30)).max())
    assert frac > 0.02, frac
