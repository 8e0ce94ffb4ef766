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


def attention(q, k, v, scale, causal=False, allowed=None):
    """q, k, v: nested sequences [N][d] of floats for one head. allowed(i, j) -> bool, if given,
    replaces the causal rule; a row with no allowed key gets o = 0 and lse = -inf.

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
            if allowed is not None:
                keys = [j for j in range(n) if allowed(i, j)]
            else:
                keys = range(i + 1) if causal else range(n)
            if not keys:
                out.append([0.0] * d)
                lses.append(float("-inf"))
                continue
            e = {}
            for j in keys:
                dot = sum((qi[c] * kd[j][c] for c in range(d)), Decimal(0))
                e[j] = (sc * dot).exp()
            z = sum(e.values(), Decimal(0))
            out.append([float(sum((e[j] * vd[j][c] for j in keys), Decimal(0)) / z) for c in range(d)])
            lses.append(float(z.ln()))
    return out, lses


def _outputs(qd, kd, vd, sc, causal, allowed=None):
    """The definition in Decimal: o [N][d] for Decimal inputs (no conversion, no rounding to float).
    allowed(i, j), if given, replaces the causal rule; a row with no allowed key gives o = 0."""
    n, d = len(qd), len(qd[0])
    out = []
    for i in range(n):
        keys = [j for j in range(n) if allowed(i, j)] if allowed is not None else (range(i + 1) if causal else range(n))
        if not keys:
            out.append([Decimal(0)] * d)
            continue
        e = {}
        for j in keys:
            e[j] = (sc * sum((qd[i][c] * kd[j][c] for c in range(d)), Decimal(0))).exp()
        z = sum(e.values(), Decimal(0))
        out.append([sum((e[j] * vd[j][c] for j in keys), Decimal(0)) / z for c in range(d)])
    return out


def loss_gradients(q, k, v, dout, scale, causal=False, h="1e-20", allowed=None):
    """Gradients of L = sum_ic dout[i][c] * o[i][c] with respect to q, k and v, by central
    differences of the definition in 50-digit arithmetic: dL/dx = (L(x+h) - L(x-h)) / 2h.

    No chain rule is used, so this checks the analytic gradients independently. With h = 1e-20
    the truncation error is of order h^2 and the cancellation error of order 1e-50 / h, both far
    below fp64 resolution. Inputs are nested sequences [N][d] of floats for one head; returns
    (dq, dk, dv) as nested lists of Python floats. allowed(i, j), if given, replaces the causal
    rule (the loss then runs over the allowed pairs only).
    """
    with localcontext() as ctx:
        ctx.prec = 50
        sc = Decimal(float(scale))
        hd = Decimal(h)
        base = [[[Decimal(float(x)) for x in row] for row in t] for t in (q, k, v)]
        go = [[Decimal(float(x)) for x in row] for row in dout]

        def loss(tensors):
            o = _outputs(tensors[0], tensors[1], tensors[2], sc, causal, allowed)
            return sum((go[i][c] * o[i][c] for i in range(len(o)) for c in range(len(o[0]))), Decimal(0))

        grads = []
        for which in range(3):
            g = []
            for i in range(len(base[which])):
                row = []
                for c in range(len(base[which][0])):
                    x0 = base[which][i][c]
                    base[which][i][c] = x0 + hd
                    lp = loss(base)
                    base[which][i][c] = x0 - hd
                    lm = loss(base)
                    base[which][i][c] = x0
                    row.append(float((lp - lm) / (2 * hd)))
                g.append(row)
            grads.append(g)
    return tuple(grads)
