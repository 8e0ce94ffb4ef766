"""Backward on tiny and sharply peaked heads, against the fp64 oracle under an elementwise bound
that follows the kernels' arithmetic.

The per-head rule of tests/test_gpu_backward.py (error within 4 unit roundoffs of the head's
largest gradient) is set for the workloads' shapes. On a head of a few keys, or with a window of
a few keys and wide logits, a gradient can be small against the terms that cancel in it, and the
operand roundings the kernels make by design show at that scale. For dq the sum is
dq_i = scale * sum_j dS_ij k_j with dS_ij = P_ij (dP_ij - D_i), and the kernels:
  - round dS to the input dtype as the operand of the dQ and dK products (|error| <= u |dS_ij|);
  - take P from the forward's lse, whose own rounding moves P by up to about u relative, which
    moves dS by up to u |dS_ij|;
  - compute D_i = dO_i . O_i from the stored O, rounded to the input dtype (|error| <= u A_i,
    A_i = sum_c |dO_ic| |O_ic|), which moves dS_ij by up to P_ij u A_i.
So per element |dq_gpu - dq_ref| <= scale * u * (2 sum_j |dS_ij| |k_jc| + A_i sum_j P_ij |k_jc|),
and the same with q for dk; dv_j = sum_i P_ij dO_i with P rounded as an operand and taken from
the forward's lse: u * 2 sum_i P_ij |dO_ic|. In f16, P and dS below 2^-14 are subnormal, where
rounding is absolute (at most 2^-25) rather than relative: each allowed pair adds that much times
|k_jc| (dq, with scale), |q_ic| (dk, with scale) or |dO_ic| (dv). Each bound is doubled (fp32
accumulation, the exp2 approximation) and allows half an output ulp. u is the unit roundoff:
2^-11 (f16), 2^-8 (bf16).
The cases include the shapes a randomized sweep found beyond the per-head rule.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import core
from _compare import ulp

pytestmark = pytest.mark.gpu

UNIT = {"f16": 2.0**-11, "bf16": 2.0**-8}
SUBNORMAL_HALF_STEP = {"f16": 2.0**-25, "bf16": 2.0**-134}


def _allowed(N, b, wl, wr, seqlens):
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    a = np.ones((N, N), dtype=bool)
    if wl >= 0:
        a &= j >= i - wl
    if wr >= 0:
        a &= j <= i + wr
    if seqlens is not None:
        a &= j < seqlens[b]
    return a


def _bounds(q, k, v, dout, scale, wl, wr, seqlens, dt):
    """Elementwise bounds on dq, dk, dv (fp64, [G, N, d]) from the module docstring."""
    B, H, N, d = q.shape
    u = UNIT[dt]
    sub = SUBNORMAL_HALF_STEP[dt]
    out = []
    for g in range(B * H):
        b = g // H
        Q, K, V, dO = (x.reshape(B * H, N, d)[g].double().numpy() for x in (q, k, v, dout))
        allowed = _allowed(N, b, wl, wr, seqlens)
        s = np.where(allowed, scale * Q @ K.T, -np.inf)
        mx = s.max(axis=1, keepdims=True)
        mx = np.where(np.isfinite(mx), mx, 0.0)
        e = np.exp(s - mx)
        l = e.sum(axis=1, keepdims=True)
        P = np.where(l > 0, e / np.where(l > 0, l, 1.0), 0.0)
        O = P @ V
        D = (dO * O).sum(axis=1, keepdims=True)
        dS = P * (dO @ V.T - D)
        A = (np.abs(dO) * np.abs(O)).sum(axis=1, keepdims=True)
        W = allowed.astype(np.float64)
        bq = scale * (u * (2 * np.abs(dS) @ np.abs(K) + A * (P @ np.abs(K))) + sub * W @ np.abs(K))
        bk = scale * (u * (2 * np.abs(dS).T @ np.abs(Q) + (P * A).T @ np.abs(Q)) + sub * W.T @ np.abs(Q))
        bv = u * 2 * P.T @ np.abs(dO) + sub * W.T @ np.abs(dO)
        out.append((2 * bq, 2 * bk, 2 * bv))
    return [np.stack([o[i] for o in out]) for i in range(3)]


# (B, H, N, d, dtype, sigma of q and k, window_left, window_right, key lengths)
CASES = [
    (2, 1, 5, 64, "f16", 3.0, 7, 0, [5, 2]),
    (1, 2, 13, 64, "f16", 3.0, 5, 0, None),
    (2, 1, 29, 128, "bf16", 3.0, -1, 22, [2, 11]),
    (2, 2, 4, 128, "bf16", 1.0, -1, 0, None),
    (1, 2, 212, 128, "f16", 3.0, 3, 0, None),
    (1, 1, 1, 64, "bf16", 3.0, -1, -1, None),
    (1, 3, 7, 128, "f16", 3.0, -1, -1, None),
    (2, 2, 40, 64, "bf16", 3.0, 0, 0, [40, 17]),
    (1, 2, 300, 128, "f16", 3.0, 1, 1, None),
    (1, 2, 2, 64, "bf16", 3.0, 1, 2, None),
    (1, 2, 35, 128, "bf16", 3.0, 2, 0, None),
]


@pytest.mark.parametrize("B,H,N,d,dt,sigma,wl,wr,seqlens", CASES)
def test_tiny_and_peaked_heads_within_the_rounding_bound(B, H, N, d, dt, sigma, wl, wr, seqlens):
    import exact_tiled_softmax_fa_amd as fa
    q, k, v = workloads.custom_inputs(B, H, N, d, dt, 8000 + N + d, sigma_qk=sigma)
    dout = workloads.custom_inputs(B, H, N, d, dt, 8001 + N + d)[0]
    scale = float(np.float32(1 / np.sqrt(d)))
    qc, kc, vc, dc = (t.cuda() for t in (q, k, v, dout))
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    o, lse = fa.forward_masked(qc, kc, vc, wl, wr, sl, scale=scale)
    grads = fa.backward_masked(qc, kc, vc, o, lse, dc, wl, wr, sl, scale=scale)
    torch.cuda.synchronize()
    refs = core.attention_backward_masked(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                          dout.double().numpy(), scale, wl, wr, seqlens)[:3]
    bounds = _bounds(q, k, v, dout, scale, wl, wr, seqlens, dt)
    G = B * H
    for name, g, r, bnd in zip(("dq", "dk", "dv"), grads, refs, bounds):
        got = g.float().cpu().double().numpy().reshape(G, N, d)
        ref = np.asarray(r).reshape(G, N, d)
        err = np.abs(got - ref)
        lim = bnd + 0.5 * ulp(ref, dt) + 1e-30
        worst = float((err / lim).max())
        print(f"[bwd edges] {name}: worst error / bound = {worst:.3f}", flush=True)
        assert np.all(err <= lim), f"{name}: {int(np.sum(err > lim))} elements over the bound (worst {worst:.3f})"
