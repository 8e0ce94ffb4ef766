"""A CPU model of the forward kernel's designed roundings states why the bf16 kernels keep the exact
running maximum ("transformer math: flash attention math", aicassindra.com, "The block-wise update,
and the full algorithm") while the f16 kernels may move the reference lazily.

The model follows the kernel per 64-key tile: scores in fp32; p = exp2(s c - m c) with
c = scale log2(e); p rounded to the input dtype as the second product's operand; the row sums
(by the four 16-key groups a lane holds) of the rounded p, which also normalise O under the lazy
reference (the f16 kernels), and of the unrounded p, which normalise O under the exact maximum
(the bf16 kernels); O = (sum p~ v) / l in fp32, stored rounded to the dtype. Reference policies:
  lazy   the wave's 32 rows keep a reference m that moves only when some group sum of some row
         exceeds 2^tau (tau = 8), and then to the tile max + tau/2 (all rows of the wave move);
  exact  m is each row's running maximum, moved whenever a tile's max exceeds it.
In bf16 (8 significant bits) every rounded p is off by up to 2^-8 of itself; against the exact
maximum a row's largest weight is exactly 1, against the lazy reference it is not, so when two or
three keys share a row's weight their errors no longer partly cancel. On the input a randomized GPU
sweep caught (B2-H1-N2214-d128, q and k with standard deviation 3, seed 1048243725: one element
1.0210e-2 from the fp64 oracle at |O| = 1.049 under the lazy reference), the model reproduces that
value to about 1e-7 and puts the exact maximum well inside the bound. Only the wave of 32 rows
holding that element is modelled (waves are independent). Runs without a GPU.
"""
import numpy as np

import workloads
from oracle import core


def _round(x, dt):
    x = np.asarray(x, dtype=np.float32)
    if dt == "f16":
        return x.astype(np.float16).astype(np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def model_forward_wave(Q, K, V, scale, dt, policy, tau=8.0):
    """O (stored, fp64 [R, d]) of one wave's rows Q [R, d] against all keys K, V [N, d]."""
    R, d = Q.shape
    N = K.shape[0]
    c = np.float32(np.float32(scale) * np.float32(1.4426950408889634))
    S = (Q @ K.T).astype(np.float32)
    tau_raw = np.float32(np.float32(tau) / c)
    headroom = np.float32(0.5) * tau_raw if policy == "lazy" else np.float32(0)
    p_cap = np.float32(2.0 ** tau)
    m = np.full(R, -np.inf, np.float32)
    mc = np.zeros(R, np.float32)
    l_run = np.zeros(R, np.float32)
    O = np.zeros((R, d), np.float32)
    group = (np.arange(64) // 4) % 4  # the lane group holding each key of a tile

    def move(mx, rows):
        nonlocal m, mc, l_run, O
        m_new = np.where(rows, np.maximum(m, (mx + headroom).astype(np.float32)), m)
        with np.errstate(invalid="ignore"):
            alpha = np.where(m_new != m, np.exp2(((m - m_new) * c).astype(np.float32)), np.float32(1))
        alpha = np.where(np.isnan(alpha), np.float32(0), alpha).astype(np.float32)
        O = (O * alpha[:, None]).astype(np.float32)
        l_run = (l_run * alpha).astype(np.float32)
        m = m_new
        mc = np.where(m == -np.inf, np.float32(0), (m * c).astype(np.float32))

    def exps(s):
        p = np.exp2((s.astype(np.float64) * c - mc[:, None].astype(np.float64)).astype(np.float32))
        pr = _round(p.astype(np.float32), dt)
        summed = pr if policy == "lazy" else p.astype(np.float32)
        sums = np.stack([summed[:, group == g].astype(np.float64).sum(1) for g in range(4)], 1).astype(np.float32)
        return pr, sums

    for k0 in range(0, N, 64):
        hi = min(N, k0 + 64)
        s = np.full((R, 64), -np.inf, np.float32)
        s[:, :hi - k0] = S[:, k0:hi]
        vt = np.zeros((64, d))
        vt[:hi - k0] = V[k0:hi]
        mx = s.max(1)
        if policy == "exact":
            move(mx, np.ones(R, bool))
            pr, sums = exps(s)
        else:
            if k0 == 0:
                move(mx, np.ones(R, bool))
            pr, sums = exps(s)
            if (sums > p_cap).any():  # a ballot over the wave: every row moves
                move(mx, np.ones(R, bool))
                pr, sums = exps(s)
        l_run = (l_run + sums.astype(np.float64).sum(1)).astype(np.float32)
        O = (O.astype(np.float64) + pr.astype(np.float64) @ vt).astype(np.float32)
    return _round((O / l_run[:, None]).astype(np.float32), dt).astype(np.float64)


def _case_wave():
    B, H, N, d, dt = 2, 1, 2214, 128, "bf16"
    q, k, v = workloads.custom_inputs(B, H, N, d, dt, 1048243725, sigma_qk=3.0)
    scale = float(np.float32(1 / np.sqrt(d)))
    bh, rows = 1, np.arange(576, 608)  # the wave (rows 32 * 18 ..) of head 1 holding the element
    Q, K, V = (t.double().numpy().reshape(B * H, N, d)[bh] for t in (q, k, v))
    o_ref, _ = core.attention(Q[None, None], K[None, None], V[None, None], scale, False, rows[None, :])
    return Q[rows], K, V, scale, np.asarray(o_ref).reshape(len(rows), d)


def test_lazy_reference_reproduces_the_bf16_miss():
    Q, K, V, scale, ref = _case_wave()
    err = np.abs(model_forward_wave(Q, K, V, scale, "bf16", "lazy") - ref)
    i = np.unravel_index(np.argmax(err), err.shape)
    assert (i[0] + 576, i[1]) == (593, 69)
    assert abs(err[i] - 1.0210136e-2) < 1e-7 and abs(ref[i] - 1.0493) < 1e-3


def test_exact_maximum_keeps_the_wave_inside_the_bound():
    Q, K, V, scale, ref = _case_wave()
    err = np.abs(model_forward_wave(Q, K, V, scale, "bf16", "exact") - ref)
    assert err.max() < 1e-2, err.max()  # the literal bound everywhere (worst 7.8e-3 at |O| = 2.24)
    assert err[np.abs(ref) < 2].max() < 5e-3  # half the bound where rounding the output costs < 4e-3
    assert err[593 - 576, 69] < 3e-3  # the element the lazy reference put at 1.02e-2


def test_f16_lazy_reference_stays_inside_its_bound_on_the_same_logits():
    """The same peaked logits in f16 (11 significant bits): the lazy reference's extra rounding stays
    well inside the 2e-3 bound."""
    B, H, N, d = 2, 1, 2214, 128
    q, k, v = workloads.custom_inputs(B, H, N, d, "f16", 1048243725, sigma_qk=3.0)
    scale = float(np.float32(1 / np.sqrt(d)))
    rows = np.arange(576, 608)
    Q, K, V = (t.double().numpy().reshape(B * H, N, d)[1] for t in (q, k, v))
    o_ref, _ = core.attention(Q[None, None], K[None, None], V[None, None], scale, False, rows[None, :])
    err = np.abs(model_forward_wave(Q[rows], K, V, scale, "f16", "lazy") - np.asarray(o_ref).reshape(32, d))
    assert err.max() < 1.5e-3, err.max()
