"""Brute-force attention in 50-digit decimal arithmetic. Test infrastructure only.

The definition with a bare exponential and no max-subtraction ("transformer
math: flash attention math", section "What we must compute, and why storage is
the problem"): s_j = scale * (q . k_j), a_j = exp(s_j) / sum_t exp(s_t),
o = sum_j a_j v_j, and lse = ln sum_t exp(s_t). Every fp64 input converts to
Decimal exactly; with 50 significant digits the result is exact to far below
fp64 resolution for the tiny sizes it is used on (N <= 16, d <= 8). It shares
no code with the C oracle it checks.
"""
from decimal import Decimal, localcontext


def attention(q, k, v, scale, causal=False):
    """q, k, v: nested sequences [N][d] of floats for one head.

    Returns (o, lse) as lists of Python floats: o [N][d], lse [N].
    """
    n = len(q)
    d = len(q[0])
    out, lses = [], []
    with localcontext() as ctx:
        ctx.prec = 50
        sc = Decimal(float(scale))
        kd = [[Decimal(float(x)) for x in row] for row in k]
        vd = [[Decimal(float(x)) for x in row] for row in v]
        for i in range(n):
            qi = [Decimal(float(x)) for x in q[i]]
            keys = range(i + 1) if causal else range(n)
            e = {}
            for j in keys:
                dot = sum((qi[c] * kd[j][c] for c in range(d)), Decimal(0))
                e[j] = (sc * dot).exp()
            z = sum(e.values(), Decimal(0))
            out.append([float(sum((e[j] * vd[j][c] for j in keys), Decimal(0)) / z) for c in range(d)])
            lses.append(float(z.ln()))
    return out, lses
