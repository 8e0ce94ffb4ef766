"""Pins of the block-sparse backward oracle (``core.attention_backward_blocksparse``).

None uses the chain rule the oracle implements:
- 50-digit central differences of the block-masked forward definition (``brute.loss_gradients``
  with the same predicate), block sizes that do not divide N, rows without keys included;
- fp64 autograd through a materialised softmax under the same block mask, per-head masks;
- reductions: an all-ones mask is the masked gradient oracle; a block-diagonal mask is the
  unmasked gradient of each block on its own;
- sum rules (dk sums to 0, dv to dout over the rows that keep a key) and zero cases.
"""
import numpy as np
import pytest
import torch

from oracle import brute, core


def _rand(seed, *shape, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


def _mask(seed, shape, p):
    return (np.random.default_rng(seed).random(shape) < p).astype(np.uint8)


@pytest.mark.parametrize("N,d,bq,bk,wl,wr,seed", [
    (7, 2, 2, 3, -1, -1, 0), (8, 2, 3, 2, 2, 1, 1), (6, 3, 4, 4, -1, 0, 2), (7, 2, 1, 2, -1, -1, 3),
])
def test_match_decimal_finite_differences(N, d, bq, bk, wl, wr, seed):
    q, k, v, do = (_rand(seed + 10 * t, 1, 1, N, d, sigma=1.5) for t in range(4))
    m = _mask(200 + seed, (-(-N // bq), -(-N // bk)), 0.6)
    dq, dk, dv, lse, delta = core.attention_backward_blocksparse(q, k, v, do, 0.7, m, bq, bk, wl, wr)

    def allowed(i, j):
        return bool(m[i // bq, j // bk]) and (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr)

    bq_, bk_, bv_ = brute.loss_gradients(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.7, allowed=allowed)
    for got, want in ((dq[0], bq_), (dk[0], bk_), (dv[0], bv_)):
        np.testing.assert_allclose(got, np.array(want), rtol=1e-9, atol=1e-11)


def test_match_torch_autograd_fp64():
    B, H, N, d, bq, bk = 2, 3, 20, 4, 4, 6
    q, k, v, do = (_rand(300 + t, B, H, N, d) for t in range(4))
    m = _mask(310, (H, 5, 4), 0.55)
    dq, dk, dv, _, _ = core.attention_backward_blocksparse(q, k, v, do, 0.6, m, bq, bk)
    t = [torch.tensor(a, requires_grad=True) for a in (q, k, v)]
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    allowed = torch.tensor(m)[:, i // bq, j // bk].bool()[None]  # [1, H, N, N]
    s = (0.6 * t[0] @ t[1].transpose(-1, -2)).masked_fill(~allowed, float("-inf"))
    keep = allowed.any(-1, keepdim=True)
    mx = torch.where(keep, s.amax(-1, keepdim=True), torch.zeros((), dtype=torch.float64))
    e = torch.exp(s - mx)
    p = torch.where(keep, e / e.sum(-1, keepdim=True).clamp_min(1e-300), torch.zeros((), dtype=torch.float64))
    ((p @ t[2]) * torch.tensor(do)).sum().backward()
    for got, x in ((dq, t[0]), (dk, t[1]), (dv, t[2])):
        np.testing.assert_allclose(got.reshape(B, H, N, d), x.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_reductions():
    q, k, v, do = (_rand(320 + t, 2, 2, 30, 3) for t in range(4))
    got = core.attention_backward_blocksparse(q, k, v, do, 0.5, np.ones((4, 3)), 8, 10, 5, 2, [30, 21])
    want = core.attention_backward_masked(q, k, v, do, 0.5, 5, 2, [30, 21])
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)
    L = 10
    got = core.attention_backward_blocksparse(q, k, v, do, 0.5, np.eye(3), L, L)
    for b0 in range(0, 30, L):
        sub = core.attention_backward(*(a[:, :, b0:b0 + L] for a in (q, k, v, do)), 0.5)
        for a, b in zip(got[:3], sub[:3]):
            np.testing.assert_allclose(a.reshape(2, 2, 30, 3)[:, :, b0:b0 + L].reshape(b.shape), b,
                                       rtol=1e-12, atol=1e-14)


def test_sum_rules_and_zero_cases():
    B, H, N, d = 1, 2, 24, 3
    q, k, v, do = (_rand(330 + t, B, H, N, d) for t in range(4))
    m = np.ones((3, 4), dtype=np.uint8)
    m[1] = 0       # rows 8..15 keep no key
    m[:, 3] = 0    # keys 18..23 are allowed to no row
    dq, dk, dv, lse, delta = core.attention_backward_blocksparse(q, k, v, do, 0.5, m, 8, 6)
    for g in range(B * H):
        np.testing.assert_allclose(dk[g].sum(0), 0.0, atol=1e-12)
        keep = np.isfinite(lse[g])
        np.testing.assert_allclose(dv[g].sum(0), do.reshape(B * H, N, d)[g][keep].sum(0), atol=1e-12)
    assert np.all(np.isneginf(lse[:, 8:16])) and np.all(dq[:, 8:16] == 0.0) and np.all(delta[:, 8:16] == 0.0)
    assert np.all(dk[:, 18:] == 0.0) and np.all(dv[:, 18:] == 0.0)
    with pytest.raises(ValueError):
        core.attention_backward_blocksparse(q, k, v, do, 0.5, np.ones((2, 4)), 8, 6)
