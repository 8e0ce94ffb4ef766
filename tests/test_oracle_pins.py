"""Pins of the fp64 CPU oracle against what the pages and mathematics fix.

Every check here is independent of the oracle's own code path: printed worked
examples, closed forms, invariants, and a 50-digit brute force. Each of the
four implementation mistakes the pages warn about is planted in the recurrence
model and must make at least one of these checks fail.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import brute, core, recurrence

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _scores_as_attention(scores, values=None, extra_dims=0):
    """A one-head problem whose logits equal ``scores`` exactly: d = 1 + extra_dims,
    q = e_0, k_j = scores_j * e_0, scale = 1."""
    n = len(scores)
    d = 1 + extra_dims
    q = np.zeros((1, 1, n, d))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, n, d))
    k[0, 0, :, 0] = scores
    if values is None:
        v = np.zeros((1, 1, n, d))
    else:
        v = np.asarray(values, dtype=np.float64).reshape(1, 1, n, -1)
    return q, k, v


# --- worked example, four keys (aicassindra.com, "A fully worked numeric example") ---

def test_worked_example_four_keys_oracle():
    g = _load("worked_example_four_keys.json")
    s = np.array(g["scores"])
    q, k, v = _scores_as_attention(s, g["values"])
    # only row 0's query matters; every row has the same q so all rows agree
    o, lse = core.attention(q, k, v, 1.0)
    assert abs(o[0, 0, 0, 0] - g["o"]["value"]) <= g["o"]["tol"]
    m = max(g["scores"])
    l = math.exp(lse[0, 0, 0] - m)
    assert abs(l - g["l"]["value"]) <= g["l"]["tol"]
    assert abs(o[0, 0, 0, 0] * l - g["o_tilde"]["value"]) <= g["o_tilde"]["tol"]
    # the weights: with V = identity the output row is the softmax row itself
    q4, k4, _ = _scores_as_attention(s, None, extra_dims=3)
    o4, lse4 = core.attention(q4, k4, np.eye(4).reshape(1, 1, 4, 4), 1.0)
    w = o4[0, 0, 0] * math.exp(lse4[0, 0, 0] - m)
    assert np.all(np.abs(w - np.array(g["weights_against_max"]["value"])) <= g["weights_against_max"]["tol"])


def test_worked_example_four_keys_recurrence_trace():
    g = _load("worked_example_four_keys.json")
    o, trace = recurrence.online_softmax(g["scores"], g["values"], g["blocks"])
    assert abs(o - g["o"]["value"]) <= g["o"]["tol"]
    for st, ref in zip(trace, g["trace"]):
        tol = ref["tol"]
        assert st["m"] == ref["m"]
        assert abs(st["alpha"] - ref["alpha"]) <= tol
        assert np.all(np.abs(st["p"] - np.array(ref["p"])) <= tol)
        assert abs(st["l"] - ref["l"]) <= tol
        assert abs(st["o_tilde"][0] - ref["o_tilde"]) <= tol
    # first block starts from m = -inf: alpha is exactly 0
    assert trace[0]["alpha"] == 0.0
    # reversed block order: same final output (order never enters the result)
    o_rev, _ = recurrence.online_softmax(g["scores"], g["values"], g["blocks"][::-1])
    assert abs(o_rev - o) <= 1e-12 * abs(o)


# --- worked example, eight scores (bibekananda.in, "Online softmax") ---

def test_worked_example_eight_scores_recurrence():
    g = _load("worked_example_eight_scores.json")
    _, trace = recurrence.online_softmax(g["scores"], np.zeros(8), g["blocks"])
    tol = g["running_sum"]["tol"]
    for st, m_ref, l_ref in zip(trace, g["running_max"], g["running_sum"]["value"]):
        assert st["m"] == m_ref
        assert abs(st["l"] - l_ref) <= tol


def test_worked_example_eight_scores_oracle():
    g = _load("worked_example_eight_scores.json")
    s = np.array(g["scores"])
    tol = g["running_sum"]["tol"]
    for upto, m_ref, l_ref in zip((4, 8), g["running_max"], g["running_sum"]["value"]):
        q, k, v = _scores_as_attention(s[:upto])
        _, lse = core.attention(q, k, v, 1.0)
        assert abs(math.exp(lse[0, 0, 0] - m_ref) - l_ref) <= tol


# --- invariants and closed forms ---

def _rand(shape, rng, sigma=1.0):
    return rng.standard_normal(shape) * sigma


@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(causal):
    rng = np.random.default_rng(7)
    n = 24
    q, k = _rand((2, 3, n, n), rng), _rand((2, 3, n, n), rng)
    v = np.broadcast_to(np.eye(n), (2, 3, n, n)).copy()
    o, _ = core.attention(q, k, v, 0.3, causal=causal)
    assert np.all(o >= 0)
    assert np.max(np.abs(o.sum(-1) - 1.0)) <= 1e-14
    if causal:
        # future keys carry no weight
        assert np.all(np.triu(o, 1) == 0)
    ones = np.ones((2, 3, n, 5))
    o1, _ = core.attention(_rand((2, 3, n, 5), rng), _rand((2, 3, n, 5), rng), ones, 0.7, causal=causal)
    assert np.max(np.abs(o1 - 1.0)) <= 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_shift_invariance(causal):
    """Adding c_i to every logit of row i leaves o_i unchanged and adds c_i to lse_i.
    Built with an extra channel: q_i[-1] = c_i / scale, k_j[-1] = 1."""
    rng = np.random.default_rng(11)
    B, H, n, d = 1, 2, 40, 6
    scale = 0.25
    q, k, v = _rand((B, H, n, d), rng), _rand((B, H, n, d), rng), _rand((B, H, n, d), rng)
    c = rng.uniform(-50, 50, size=(B, H, n))
    q2 = np.concatenate([q, (c / scale)[..., None]], axis=-1)
    k2 = np.concatenate([k, np.ones((B, H, n, 1))], axis=-1)
    v2 = np.concatenate([v, np.zeros((B, H, n, 1))], axis=-1)
    o, lse = core.attention(q, k, v, scale, causal=causal)
    o2, lse2 = core.attention(q2, k2, v2, scale, causal=causal)
    assert np.max(np.abs(o2[..., :d] - o)) <= 1e-12
    assert np.max(np.abs(lse2 - (lse + c))) <= 1e-11


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_keys_give_mean_of_values(causal):
    rng = np.random.default_rng(3)
    n, d = 33, 8
    q = _rand((1, 2, n, d), rng)
    k = np.zeros((1, 2, n, d))
    v = _rand((1, 2, n, d), rng)
    o, lse = core.attention(q, k, v, 0.125, causal=causal)
    for i in range(n):
        cnt = i + 1 if causal else n
        assert np.allclose(o[:, :, i], v[:, :, :cnt].mean(axis=2), rtol=0, atol=1e-14)
        assert np.allclose(lse[:, :, i], math.log(cnt), rtol=0, atol=1e-14)


def test_single_key_and_causal_row_zero():
    rng = np.random.default_rng(5)
    d = 16
    scale = float(np.float32(1 / math.sqrt(d)))
    q, k, v = _rand((2, 2, 1, d), rng), _rand((2, 2, 1, d), rng), _rand((2, 2, 1, d), rng)
    o, lse = core.attention(q, k, v, scale)
    assert np.array_equal(o, v)
    assert np.allclose(lse, scale * np.sum(q * k, -1), rtol=0, atol=1e-13)
    n = 50
    q, k, v = _rand((1, 3, n, d), rng), _rand((1, 3, n, d), rng), _rand((1, 3, n, d), rng)
    o, lse = core.attention(q, k, v, scale, causal=True)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    assert np.allclose(lse[:, :, 0], scale * np.sum(q[:, :, 0] * k[:, :, 0], -1), rtol=0, atol=1e-13)


def test_large_logits_do_not_overflow():
    """Logits far beyond ln(DBL_MAX) = 709.8: a bare exp would overflow to inf, the
    max-subtracted form must not (aicassindra.com, "Proof of numerical stability")."""
    rng = np.random.default_rng(9)
    n, d = 12, 4
    q = _rand((1, 1, n, d), rng, 30.0)
    k = _rand((1, 1, n, d), rng, 30.0)
    v = _rand((1, 1, n, d), rng)
    o, lse = core.attention(q, k, v, 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.max(np.abs(lse)) > 800  # the case really is past the fp64 exp range
    ob, lb = brute.attention(q[0, 0], k[0, 0], v[0, 0], 1.0)
    assert np.max(np.abs(o[0, 0] - np.array(ob))) <= 1e-12
    assert np.max(np.abs(lse[0, 0] - np.array(lb)) / np.abs(np.array(lb))) <= 1e-14


@pytest.mark.parametrize("n,d,causal,sigma", [
    (1, 1, False, 1.0), (2, 3, False, 1.0), (3, 2, True, 1.0), (5, 4, False, 3.0),
    (8, 8, True, 1.0), (16, 8, False, 1.0), (16, 4, True, 4.0), (11, 7, False, 0.1),
])
def test_brute_force_tiny(n, d, causal, sigma):
    rng = np.random.default_rng(1000 + 17 * n + d)
    scale = 1 / math.sqrt(d)
    q, k, v = _rand((1, 1, n, d), rng, sigma), _rand((1, 1, n, d), rng, sigma), _rand((1, 1, n, d), rng)
    o, lse = core.attention(q, k, v, scale, causal=causal)
    ob, lb = brute.attention(q[0, 0], k[0, 0], v[0, 0], scale, causal=causal)
    ob, lb = np.array(ob), np.array(lb)
    vmax = np.max(np.abs(v))
    assert np.max(np.abs(o[0, 0] - ob)) <= 1e-13 * vmax
    assert np.max(np.abs(lse[0, 0] - lb)) <= 1e-13 * max(1.0, np.max(np.abs(lb)))


def test_row_subset_matches_full():
    rng = np.random.default_rng(21)
    B, H, n, d = 2, 2, 37, 8
    q, k, v = _rand((B, H, n, d), rng), _rand((B, H, n, d), rng), _rand((B, H, n, d), rng)
    rows = np.stack([rng.choice(n, size=5, replace=False) for _ in range(B * H)])
    for causal in (False, True):
        o, lse = core.attention(q, k, v, 0.3, causal=causal)
        os_, ls_ = core.attention(q, k, v, 0.3, causal=causal, rows=rows)
        of, lf = o.reshape(B * H, n, d), lse.reshape(B * H, n)
        for bh in range(B * H):
            assert np.array_equal(os_[bh], of[bh, rows[bh]])
            assert np.array_equal(ls_[bh], lf[bh, rows[bh]])


def test_bad_arguments_rejected():
    q = np.zeros((1, 1, 4, 2))
    with pytest.raises(RuntimeError):
        core.attention(q, q, q, 1.0, rows=np.array([[0, 4]]))
    with pytest.raises(ValueError):
        core.attention(q, q, np.zeros((1, 1, 4, 3)), 1.0)


# --- the recurrence: block order and size never enter the result ---

@pytest.mark.parametrize("seed", range(6))
def test_recurrence_partition_and_order_invariance(seed):
    rng = np.random.default_rng(seed)
    n, d = int(rng.integers(1, 90)), int(rng.integers(1, 9))
    sigma = [1.0, 5.0, 20.0][seed % 3]
    q, k, v = _rand((1, 1, n, d), rng, sigma), _rand((1, 1, n, d), rng, sigma), _rand((1, 1, n, d), rng)
    scale = 1 / math.sqrt(d)
    o_ref, _ = core.attention(q, k, v, scale)
    i = int(rng.integers(0, n))
    s = scale * (k[0, 0] @ q[0, 0, i])
    for _ in range(5):
        cuts = np.sort(rng.choice(np.arange(1, n), size=min(n - 1, int(rng.integers(0, 6))), replace=False)) if n > 1 else []
        blocks = np.split(rng.permutation(n), cuts)
        order = rng.permutation(len(blocks))
        o, _ = recurrence.online_softmax(s, v[0, 0], [blocks[t] for t in order])
        assert np.max(np.abs(o - o_ref[0, 0, i])) <= 1e-12 * max(1.0, np.max(np.abs(v)))


def test_recurrence_causal_mask_matches_oracle():
    rng = np.random.default_rng(4)
    n, d = 70, 8
    q, k, v = _rand((1, 1, n, d), rng), _rand((1, 1, n, d), rng), _rand((1, 1, n, d), rng)
    o_ref, _ = core.attention(q, k, v, 0.35, causal=True)
    for i in (0, 1, 31, 32, 69):
        s = 0.35 * (k[0, 0] @ q[0, 0, i])
        allowed = np.arange(n) <= i
        o, _ = recurrence.online_softmax(s, v[0, 0], recurrence.blocks_of(n, 16), allowed=allowed)
        assert np.max(np.abs(o - o_ref[0, 0, i])) <= 1e-13


# --- each planted mistake must be caught by one of the pins above ---

def _passes_four_key_example(pitfall):
    g = _load("worked_example_four_keys.json")
    o, _ = recurrence.online_softmax(g["scores"], g["values"], g["blocks"], pitfall=pitfall)
    return bool(abs(o - g["o"]["value"]) <= g["o"]["tol"])


def _passes_underflow_row(pitfall):
    """Every logit around -800: exp(logit) underflows to 0 in fp64 unless the
    reference max is a real score."""
    s = np.array([-800.0, -801.5, -799.25, -802.0, -800.5, -803.0])
    v = np.array([1.0, 2.0, 3.0, 4.0, 5.0, 6.0])
    q, k, vv = _scores_as_attention(s, v)
    o_ref, _ = core.attention(q, k, vv, 1.0)
    o, _ = recurrence.online_softmax(s, v, recurrence.blocks_of(6, 2), pitfall=pitfall)
    return bool(np.isfinite(o) and abs(o - o_ref[0, 0, 0, 0]) <= 1e-12)


def _passes_masked_huge_logit(pitfall):
    """Causal row 2 of 6 keys whose future keys carry logits of +1000."""
    s = np.array([0.5, -0.25, 1.0, 1000.0, 1000.0, 999.0])
    v = np.array([1.0, 2.0, 3.0, 4.0, 5.0, 6.0])
    allowed = np.arange(6) <= 2
    w = np.exp(s[:3] - s[:3].max())
    ref = float(w @ v[:3] / w.sum())
    o, _ = recurrence.online_softmax(s, v, recurrence.blocks_of(6, 3), allowed=allowed, pitfall=pitfall)
    return bool(np.isfinite(o) and abs(o - ref) <= 1e-12)


def test_correct_recurrence_passes_every_check():
    assert _passes_four_key_example(None)
    assert _passes_underflow_row(None)
    assert _passes_masked_huge_logit(None)


@pytest.mark.parametrize("pitfall", recurrence.PITFALLS)
def test_each_planted_mistake_is_caught(pitfall):
    checks = [_passes_four_key_example(pitfall), _passes_underflow_row(pitfall), _passes_masked_huge_logit(pitfall)]
    assert not all(checks), f"pitfall {pitfall} slipped through every check"
