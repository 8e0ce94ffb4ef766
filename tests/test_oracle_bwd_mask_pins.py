"""Pins of the masked backward oracle (``core.attention_backward_masked``).

None of these uses the chain rule the oracle implements:
- 50-digit central differences of the masked forward definition (``brute.loss_gradients`` with
  the same allowed(i, j) predicate), rows without keys included;
- fp64 autograd through a plainly materialised masked softmax in PyTorch (CPU);
- reductions: the full mask is the unmasked oracle and the causal window the causal one;
- sum rules: dk sums to 0 over the keys, dv to the sum of dout over the rows that keep a key;
- keys past the key length get dk = dv = 0, rows with no key dq = 0, lse = -inf, D = 0;
- lse agrees with the masked forward oracle.
"""
import numpy as np
import pytest
import torch

from oracle import brute, core


def _rand(seed, *shape, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


def _allowed(wl, wr, L):
    return lambda i, j: (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr) and j < L


@pytest.mark.parametrize("N,d,wl,wr,L,seed", [
    (6, 2, 1, 1, 6, 0), (7, 3, -1, 2, 5, 1), (6, 2, 2, 0, 4, 2), (5, 2, 0, -1, 3, 3), (6, 3, 1, 0, 6, 4),
])
def test_match_decimal_finite_differences(N, d, wl, wr, L, seed):
    q, k, v, do = (_rand(seed + 10 * t, 1, 1, N, d, sigma=1.5) for t in range(4))
    dq, dk, dv, lse, delta = core.attention_backward_masked(q, k, v, do, 0.7, wl, wr, [L])
    bq, bk, bv = brute.loss_gradients(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.7, allowed=_allowed(wl, wr, L))
    for got, want in ((dq[0], bq), (dk[0], bk), (dv[0], bv)):
        np.testing.assert_allclose(got, np.array(want), rtol=1e-9, atol=1e-11)


def _torch_reference(q, k, v, do, scale, wl, wr, seqlens):
    B, H, N, d = q.shape
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v)]
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    s = scale * t[0] @ t[1].transpose(-1, -2)
    allowed = torch.ones(B, 1, N, N, dtype=torch.bool)
    if wl >= 0:
        allowed &= (j >= i - wl)
    if wr >= 0:
        allowed &= (j <= i + wr)
    if seqlens is not None:
        allowed &= (j[None] < torch.tensor(seqlens)[:, None, None, None])
    s = s.masked_fill(~allowed, float("-inf"))
    keep = allowed.any(-1, keepdim=True)  # rows with a key
    m = torch.where(keep, s.amax(-1, keepdim=True), torch.zeros(()))
    e = torch.exp(s - m)
    p = torch.where(keep, e / e.sum(-1, keepdim=True).clamp_min(1e-300), torch.zeros(()))
    o = p @ t[2]
    (o * torch.tensor(do)).sum().backward()
    return [x.grad.numpy() for x in t]


@pytest.mark.parametrize("wl,wr,seqlens", [(3, 2, None), (-1, 0, [20, 13]), (5, -1, [0, 20]), (0, 0, [17, 9])])
def test_match_torch_autograd_fp64(wl, wr, seqlens):
    B, H, N, d = 2, 2, 20, 4
    q, k, v, do = (_rand(50 + t, B, H, N, d) for t in range(4))
    dq, dk, dv, _, _ = core.attention_backward_masked(q, k, v, do, 0.6, wl, wr, seqlens)
    rq, rk, rv = _torch_reference(q, k, v, do, 0.6, wl, wr, seqlens)
    for got, want in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(got.reshape(want.shape), want, rtol=1e-10, atol=1e-12)


def test_reductions_to_the_unmasked_and_causal_oracles():
    q, k, v, do = (_rand(60 + t, 2, 3, 33, 5) for t in range(4))
    for (wl, wr, sl), causal in (((-1, -1, None), False), ((-1, -1, [33, 33]), False), ((-1, 0, None), True)):
        got = core.attention_backward_masked(q, k, v, do, 0.4, wl, wr, sl)
        want = core.attention_backward(q, k, v, do, 0.4, causal=causal)
        for a, b in zip(got, want):
            np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


def test_sum_rules_and_zero_cases():
    B, H, N, d = 2, 2, 24, 3
    q, k, v, do = (_rand(70 + t, B, H, N, d) for t in range(4))
    seqlens = [15, 24]
    dq, dk, dv, lse, delta = core.attention_backward_masked(q, k, v, do, 0.5, 4, 0, seqlens)
    dq, dk, dv = (a.reshape(B, H, N, d) for a in (dq, dk, dv))
    lse, delta = lse.reshape(B, H, N), delta.reshape(B, H, N)
    has_key = np.isfinite(lse)
    for b in range(B):
        for h in range(H):
            np.testing.assert_allclose(dk[b, h].sum(0), 0.0, atol=1e-12)
            np.testing.assert_allclose(dv[b, h].sum(0), do[b, h][has_key[b, h]].sum(0), atol=1e-12)
    # batch 0: keys 15.. never allowed; rows 19.. (window 4 back, none ahead) keep no key
    assert np.all(dk[0, :, 15:] == 0.0) and np.all(dv[0, :, 15:] == 0.0)
    assert np.all(np.isneginf(lse[0, :, 19:])) and np.all(delta[0, :, 19:] == 0.0)
    assert np.all(dq[0, :, 19:] == 0.0)
    assert np.all(np.isfinite(lse[1]))


def test_lse_agrees_with_the_masked_forward():
    q, k, v, do = (_rand(80 + t, 2, 2, 40, 4) for t in range(4))
    _, _, _, lse, delta = core.attention_backward_masked(q, k, v, do, 0.3, 6, 2, [40, 11])
    o, lse_f = core.attention_masked(q, k, v, 0.3, 6, 2, [40, 11])
    np.testing.assert_allclose(lse.reshape(lse_f.shape), lse_f, rtol=1e-13)
    np.testing.assert_allclose(delta.reshape(2, 2, 40), (do * o).sum(-1), rtol=1e-10, atol=1e-12)


def test_row_and_key_subsets_and_bad_arguments():
    q, k, v, do = (_rand(90 + t, 1, 2, 30, 4) for t in range(4))
    full = core.attention_backward_masked(q, k, v, do, 0.5, 5, 5, [22])
    rows = np.array([[0, 7, 29], [3, 21, 28]])
    keys = np.array([[1, 21, 25], [0, 10, 29]])
    part = core.attention_backward_masked(q, k, v, do, 0.5, 5, 5, [22], rows=rows, keys=keys)
    for g in range(2):
        np.testing.assert_array_equal(part[0][g], full[0][g][rows[g]])
        np.testing.assert_array_equal(part[1][g], full[1][g][keys[g]])
        np.testing.assert_array_equal(part[2][g], full[2][g][keys[g]])
    with pytest.raises(RuntimeError):
        core.attention_backward_masked(q, k, v, do, 0.5, -2, 0)
    with pytest.raises(RuntimeError):
        core.attention_backward_masked(q, k, v, do, 0.5, -1, -1, [31])
    with pytest.raises(ValueError):
        core.attention_backward_masked(q, k, v, do, 0.5, -1, -1, [3, 3])
