"""Pins of the masked oracle (``core.attention_masked``): sliding windows and key padding.

The pages admit any mask that is applied to every score tile before the max ("Causal masking fits
inside the tiled computation", nalar.dev, last paragraph; aicassindra.com, "Pitfalls": masked
scores are -inf "for causal or padded attention"). Independent checks:
- the 50-digit brute force with the same allowed(i, j) predicate;
- reductions to the plain definition: every row equals unmasked attention over its own slice of
  keys [max(0, i - wl), min(len, i + wr + 1)); padding equals attention on the truncated keys;
- the masks that coincide with the two the rest of the suite pins: (-1, 0) is causal, (-1, -1) with
  full lengths is no mask;
- a row with no allowed key gives o = 0 and lse = -inf.
"""
import numpy as np
import pytest

from oracle import brute, core


def _rand(seed, B, H, N, d, sigma=1.0):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, N, d)) * (sigma if i < 2 else 1.0) for i in range(3)]


@pytest.mark.parametrize("N,d,wl,wr,seqlen,seed", [
    (9, 3, 2, 1, None, 0), (9, 3, 0, 0, None, 1), (12, 2, -1, 3, 7, 2), (12, 2, 4, -1, 10, 3),
    (7, 4, 1, 0, 5, 4), (10, 3, 3, 2, 2, 5),
])
def test_brute_force(N, d, wl, wr, seqlen, seed):
    q, k, v = _rand(seed, 1, 1, N, d, 2.0)
    sl = None if seqlen is None else [seqlen]
    o, lse = core.attention_masked(q, k, v, 0.6, wl, wr, sl)
    L = N if seqlen is None else seqlen

    def allowed(i, j):
        return (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr) and j < L

    bo, bl = brute.attention(q[0, 0], k[0, 0], v[0, 0], 0.6, allowed=allowed)
    np.testing.assert_allclose(o[0, 0], np.array(bo), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.array(bl), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("wl,wr", [(0, 0), (5, 0), (17, 3), (-1, 4), (30, -1)])
def test_rows_equal_attention_over_their_key_slice(wl, wr):
    B, H, N, d = 2, 2, 50, 8
    q, k, v = _rand(10 + max(wl, 0) + max(wr, 0), B, H, N, d)
    seqlens = [50, 37]
    o, lse = core.attention_masked(q, k, v, 0.3, wl, wr, seqlens)
    for b in range(B):
        for i in range(N):
            lo = max(0, i - wl) if wl >= 0 else 0
            hi = min(seqlens[b], i + wr + 1) if wr >= 0 else seqlens[b]
            if hi <= lo:
                assert np.all(o[b, :, i] == 0.0) and np.all(lse[b, :, i] == -np.inf)
                continue
            ks, vs = k[b, :, lo:hi], v[b, :, lo:hi]
            s = 0.3 * np.einsum("hd,hjd->hj", q[b, :, i], ks)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            expect = np.einsum("hj,hjd->hd", p, vs) / p.sum(axis=1, keepdims=True)
            np.testing.assert_allclose(o[b, :, i], expect, rtol=1e-11, atol=1e-13)
            np.testing.assert_allclose(lse[b, :, i], m[:, 0] + np.log(p.sum(axis=1)), rtol=1e-12)


def test_padding_equals_truncated_keys():
    q, k, v = _rand(20, 1, 3, 40, 6)
    L = 23
    o, lse = core.attention_masked(q, k, v, 0.5, -1, -1, [L])
    # keys past L never matter ...
    k2, v2 = k.copy(), v.copy()
    k2[:, :, L:] = 100.0
    v2[:, :, L:] = -7.0
    o2, lse2 = core.attention_masked(q, k2, v2, 0.5, -1, -1, [L])
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    # ... and the first L rows are plain attention on the first L keys
    sub_o, sub_l = core.attention(q[:, :, :L], k[:, :, :L], v[:, :, :L], 0.5)
    np.testing.assert_allclose(o[:, :, :L], sub_o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[:, :, :L], sub_l, rtol=1e-12)


def test_causal_and_no_mask_are_special_cases():
    q, k, v = _rand(30, 2, 2, 33, 5)
    oc, lc = core.attention(q, k, v, 0.4, causal=True)
    om, lm = core.attention_masked(q, k, v, 0.4, -1, 0)
    np.testing.assert_allclose(om, oc, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lm, lc, rtol=1e-13)
    on, ln = core.attention(q, k, v, 0.4)
    om, lm = core.attention_masked(q, k, v, 0.4, -1, -1, [33, 33])
    np.testing.assert_allclose(om, on, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lm, ln, rtol=1e-13)


def test_empty_rows_and_bad_arguments():
    q, k, v = _rand(40, 1, 1, 8, 2)
    o, lse = core.attention_masked(q, k, v, 1.0, 0, 0, [3])  # rows >= 3 keep no key
    assert np.all(o[0, 0, 3:] == 0.0) and np.all(np.isneginf(lse[0, 0, 3:]))
    assert np.all(np.isfinite(lse[0, 0, :3]))
    np.testing.assert_allclose(o[0, 0, :3], v[0, 0, :3])  # window 0: each row sees only itself
    with pytest.raises(RuntimeError):
        core.attention_masked(q, k, v, 1.0, -2, 0)
    with pytest.raises(RuntimeError):
        core.attention_masked(q, k, v, 1.0, -1, -1, [9])
    with pytest.raises(ValueError):
        core.attention_masked(q, k, v, 1.0, -1, -1, [3, 3])
