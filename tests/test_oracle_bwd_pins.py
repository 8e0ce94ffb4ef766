"""Pins of the fp64 backward oracle (``core.attention_backward``) against mathematics it does not use.

The pages fix the backward pass only as a dataflow (recompute tiles from saved per-row statistics),
so the values are pinned by what calculus fixes:
- 50-digit central differences of the forward definition (no chain rule anywhere), every element,
  tiny sizes, causal and not, including logits that would overflow a bare exponential in fp64;
- PyTorch autograd in fp64 on the CPU through a plain materialised softmax (an independent
  implementation of the same derivative);
- identities: the rows of dS sum to zero, so the key gradients sum to zero and adding one vector to
  every key changes no gradient; softmax rows sum to one, so the value gradients sum to the sum of
  dO; the gradients are linear in dO; closed forms for K = 0 and for N = 1;
- consistency with the forward oracle (lse) and D_i = dO_i . o_i.
"""
import numpy as np
import pytest

from oracle import brute, core


def _rand(rng, *shape, sigma=1.0):
    return rng.standard_normal(shape) * sigma


@pytest.mark.parametrize("N,d,scale,causal,sigma,seed", [
    (1, 2, 0.5, False, 1.0, 0),
    (2, 1, 1.0, True, 1.0, 1),
    (5, 3, 0.7, False, 1.0, 2),
    (5, 3, 0.7, True, 1.0, 3),
    (7, 4, 0.5, False, 2.0, 4),
    (6, 2, 1.0, True, 3.0, 5),
    (4, 3, 1.0, False, 12.0, 6),   # logits of several hundred: a bare exp would overflow in fp64
])
def test_gradients_match_decimal_finite_differences(N, d, scale, causal, sigma, seed):
    rng = np.random.default_rng(seed)
    q, k = _rand(rng, N, d, sigma=sigma), _rand(rng, N, d, sigma=sigma)
    v, do = _rand(rng, N, d), _rand(rng, N, d)
    ref = brute.loss_gradients(q, k, v, do, scale, causal)
    got = core.attention_backward(q[None], k[None], v[None], do[None], scale, causal)[:3]
    for name, r, g in zip(("dq", "dk", "dv"), ref, got):
        r = np.asarray(r)
        np.testing.assert_allclose(g[0], r, rtol=1e-12, atol=1e-13 * max(1.0, np.abs(r).max()), err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_torch_autograd_fp64(causal):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    G, N, d, scale = 3, 70, 16, 0.25
    q, k, v, do = (_rand(rng, G, N, d) for _ in range(4))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * (tq @ tk.transpose(-1, -2))
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ tv
    o.backward(torch.tensor(do, dtype=torch.float64))
    dq, dk, dv, lse, _ = core.attention_backward(q, k, v, do, scale, causal)
    for name, r, g in (("dq", tq.grad, dq), ("dk", tk.grad, dk), ("dv", tv.grad, dv)):
        np.testing.assert_allclose(g, r.numpy(), rtol=1e-11, atol=1e-13, err_msg=name)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).detach().numpy(), rtol=1e-13)


@pytest.fixture(scope="module")
def medium():
    rng = np.random.default_rng(21)
    G, N, d = 2, 300, 32
    return [_rand(rng, G, N, d) for _ in range(4)], 1 / np.sqrt(d)


@pytest.mark.parametrize("causal", [False, True])
def test_key_gradients_sum_to_zero_and_value_gradients_sum_to_dout(medium, causal):
    (q, k, v, do), scale = medium
    dq, dk, dv, _, _ = core.attention_backward(q, k, v, do, scale, causal)
    mag = np.abs(dk).max()
    assert np.abs(dk.sum(axis=1)).max() < 1e-12 * mag * q.shape[1]
    np.testing.assert_allclose(dv.sum(axis=1), do.sum(axis=1), rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("causal", [False, True])
def test_translating_every_key_changes_no_gradient(medium, causal):
    (q, k, v, do), scale = medium
    base = core.attention_backward(q, k, v, do, scale, causal)
    u = np.random.default_rng(5).standard_normal(q.shape[-1])
    moved = core.attention_backward(q, k + u, v, do, scale, causal)
    for name, a, b in zip(("dq", "dk", "dv"), base[:3], moved[:3]):
        np.testing.assert_allclose(b, a, rtol=1e-9, atol=1e-11 * np.abs(a).max(), err_msg=name)
    # the logits of row i move by scale * q_i . u, and so does its log-sum-exp
    np.testing.assert_allclose(moved[3], base[3] + scale * (q @ u), rtol=1e-12, atol=1e-12)


def test_gradients_are_linear_in_dout(medium):
    (q, k, v, do), scale = medium
    do2 = np.random.default_rng(6).standard_normal(do.shape)
    a = core.attention_backward(q, k, v, do, scale, True)
    b = core.attention_backward(q, k, v, do2, scale, True)
    c = core.attention_backward(q, k, v, 2.0 * do - 3.0 * do2, scale, True)
    for x, y, z in zip(a[:3], b[:3], c[:3]):
        np.testing.assert_allclose(z, 2.0 * x - 3.0 * y, rtol=1e-10, atol=1e-12 * np.abs(z).max())


def test_zero_keys_give_uniform_weights():
    rng = np.random.default_rng(7)
    N, d = 40, 8
    q, v, do = (_rand(rng, 1, N, d) for _ in range(3))
    k = np.zeros_like(q)
    # non-causal: every row weights every key by 1/N, so dV_j is the mean of dO, dQ is 0
    dq, dk, dv, lse, _ = core.attention_backward(q, k, v, do, 0.3, False)
    np.testing.assert_allclose(dv[0], np.broadcast_to(do[0].mean(axis=0), (N, d)), rtol=1e-13, atol=1e-14)
    assert np.abs(dq).max() == 0.0
    np.testing.assert_allclose(lse, np.log(N), rtol=1e-15)
    # causal: row i weights keys 0..i by 1/(i+1), so dV_j = sum_{i>=j} dO_i / (i+1)
    _, _, dv_c, _, _ = core.attention_backward(q, k, v, do, 0.3, True)
    w = do[0] / np.arange(1, N + 1)[:, None]
    expect = np.cumsum(w[::-1], axis=0)[::-1]
    np.testing.assert_allclose(dv_c[0], expect, rtol=1e-12, atol=1e-14)


def test_single_key():
    rng = np.random.default_rng(8)
    q, k, v, do = (_rand(rng, 4, 1, 6) for _ in range(4))
    dq, dk, dv, lse, delta = core.attention_backward(q, k, v, do, 0.5, False)
    assert np.abs(dq).max() == 0.0 and np.abs(dk).max() == 0.0
    np.testing.assert_array_equal(dv, do)
    np.testing.assert_allclose(delta, np.sum(do * v, axis=-1), rtol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_and_delta_agree_with_the_forward_oracle(medium, causal):
    (q, k, v, do), scale = medium
    _, _, _, lse, delta = core.attention_backward(q, k, v, do, scale, causal)
    o, lse_f = core.attention(q[None], k[None], v[None], scale, causal)
    np.testing.assert_array_equal(lse, lse_f[0])
    np.testing.assert_allclose(delta, np.sum(do * o[0], axis=-1), rtol=1e-11, atol=1e-13)


def test_row_and_key_subsets_match_the_full_result(medium):
    (q, k, v, do), scale = medium
    full = core.attention_backward(q, k, v, do, scale, True)
    rows = np.array([[0, 299, 17], [5, 150, 3]])
    keys = np.array([[299, 0], [42, 7]])
    dq, dk, dv, _, _ = core.attention_backward(q, k, v, do, scale, True, rows=rows, keys=keys)
    for g in range(2):
        np.testing.assert_array_equal(dq[g], full[0][g, rows[g]])
        np.testing.assert_array_equal(dk[g], full[1][g, keys[g]])
        np.testing.assert_array_equal(dv[g], full[2][g, keys[g]])


def test_bad_arguments():
    z = np.zeros((1, 4, 2))
    with pytest.raises(ValueError):
        core.attention_backward(z, z, z, np.zeros((1, 3, 2)), 1.0)
    with pytest.raises(RuntimeError):
        core.attention_backward(z, z, z, z, 1.0, rows=np.array([[4]]))
    with pytest.raises(ValueError):
        core.attention_backward(z, z, z, z, 1.0, keys=np.array([0, 1]))
