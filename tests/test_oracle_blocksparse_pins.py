"""Pins of the block-sparse oracle (``core.attention_blocksparse``).

The pages admit any mask applied to the scores before the max ("Causal masking fits inside the
tiled computation", nalar.dev, last paragraph; aicassindra.com, "Pitfalls": masked scores are
-inf). A mask over blocks of the score matrix is such a mask. Independent checks:
- the 50-digit brute force with the same allowed(i, j) predicate, block sizes that do not divide N;
- reductions to the plain definition: an all-ones mask is the general-mask oracle; a
  block-diagonal mask is independent attention inside each block; a block-lower-triangular mask
  under the causal window is causal attention;
- each row equals plain attention over exactly its allowed keys (gathered by hand);
- one mask per head or per (batch, head) agrees with the shared form when the masks are equal;
- a row with no allowed key gives o = 0 and lse = -inf.
A plausible indexing slip (row and column block swapped, a stride applied to the wrong axis, the
block index taken from the key for the row) fails the brute-force or the gather checks, since the
masks there are not symmetric and differ per head.
"""
import numpy as np
import pytest

from oracle import brute, core


def _rand(seed, B, H, N, d, sigma=1.0):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, N, d)) * (sigma if i < 2 else 1.0) for i in range(3)]


def _mask(seed, shape, p=0.5):
    return (np.random.default_rng(seed).random(shape) < p).astype(np.uint8)


@pytest.mark.parametrize("N,d,bq,bk,wl,wr,seed", [
    (9, 3, 2, 3, -1, -1, 0), (11, 2, 4, 2, -1, -1, 1), (10, 3, 3, 4, 2, 1, 2), (12, 2, 5, 3, -1, 0, 3),
    (7, 4, 1, 1, -1, -1, 4),
])
def test_brute_force(N, d, bq, bk, wl, wr, seed):
    q, k, v = _rand(seed, 1, 1, N, d, 2.0)
    n_qb, n_kb = -(-N // bq), -(-N // bk)
    m = _mask(100 + seed, (n_qb, n_kb), 0.6)
    m[:, 0] = 1  # most rows keep a key; rows that keep none are checked elsewhere
    o, lse = core.attention_blocksparse(q, k, v, 0.7, m, bq, bk, wl, wr)

    def allowed(i, j):
        return bool(m[i // bq, j // bk]) and (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr)

    bo, bl = brute.attention(q[0, 0], k[0, 0], v[0, 0], 0.7, allowed=allowed)
    bo, bl = np.array(bo, dtype=float), np.array(bl, dtype=float)
    empty = np.isneginf(bl)
    assert np.array_equal(np.isneginf(lse[0, 0]), empty)
    np.testing.assert_allclose(o[0, 0][~empty], bo[~empty], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0][~empty], bl[~empty], rtol=1e-12, atol=1e-13)
    assert np.all(o[0, 0][empty] == 0.0)


def test_all_ones_is_the_general_mask():
    q, k, v = _rand(10, 2, 2, 40, 6)
    for wl, wr, sl in ((-1, -1, None), (7, 3, [40, 29]), (-1, 0, [33, 40])):
        o, lse = core.attention_blocksparse(q, k, v, 0.4, np.ones((4, 3)), 10, 16, wl, wr, sl)
        om, lm = core.attention_masked(q, k, v, 0.4, wl, wr, sl)
        np.testing.assert_allclose(o, om, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(lse, lm, rtol=1e-13)


def test_block_diagonal_is_attention_per_block():
    B, H, N, d, L = 1, 3, 48, 5, 16
    q, k, v = _rand(11, B, H, N, d)
    o, lse = core.attention_blocksparse(q, k, v, 0.3, np.eye(N // L), L, L)
    for b0 in range(0, N, L):
        so, sl = core.attention(q[:, :, b0:b0 + L], k[:, :, b0:b0 + L], v[:, :, b0:b0 + L], 0.3)
        np.testing.assert_allclose(o[:, :, b0:b0 + L], so, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[:, :, b0:b0 + L], sl, rtol=1e-12)


def test_lower_triangular_blocks_under_the_causal_window_is_causal():
    q, k, v = _rand(12, 2, 2, 37, 4)
    tri = np.tril(np.ones((5, 5), dtype=np.uint8))  # blocks of 8: every key j <= i is in an allowed block
    o, lse = core.attention_blocksparse(q, k, v, 0.5, tri, 8, 8, -1, 0)
    oc, lc = core.attention(q, k, v, 0.5, causal=True)
    np.testing.assert_allclose(o, oc, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, lc, rtol=1e-13)


def test_rows_equal_attention_over_their_allowed_keys():
    B, H, N, d, bq, bk = 2, 2, 30, 4, 4, 7
    q, k, v = _rand(13, B, H, N, d)
    m = _mask(14, (B, H, -(-N // bq), -(-N // bk)), 0.55)
    o, lse = core.attention_blocksparse(q, k, v, 0.6, m, bq, bk, window_left=9, seqlens_k=[30, 22])
    for b in range(B):
        L = (30, 22)[b]
        for h in range(H):
            for i in range(N):
                keys = [j for j in range(max(0, i - 9), L) if m[b, h, i // bq, j // bk]]
                if not keys:
                    assert np.all(o[b, h, i] == 0.0) and lse[b, h, i] == -np.inf
                    continue
                s = 0.6 * k[b, h, keys] @ q[b, h, i]
                mx = s.max()
                p = np.exp(s - mx)
                np.testing.assert_allclose(o[b, h, i], p @ v[b, h, keys] / p.sum(), rtol=1e-11, atol=1e-13)
                np.testing.assert_allclose(lse[b, h, i], mx + np.log(p.sum()), rtol=1e-12)


def test_mask_forms_agree():
    B, H, N, d, bq, bk = 2, 3, 20, 3, 5, 4
    q, k, v = _rand(15, B, H, N, d)
    per_head = _mask(16, (H, 4, 5), 0.6)
    o_h, l_h = core.attention_blocksparse(q, k, v, 0.5, per_head, bq, bk)
    o_bh, l_bh = core.attention_blocksparse(q, k, v, 0.5, np.broadcast_to(per_head, (B, H, 4, 5)), bq, bk)
    np.testing.assert_array_equal(o_h, o_bh)
    np.testing.assert_array_equal(l_h, l_bh)
    shared = per_head[1]
    o_s, l_s = core.attention_blocksparse(q, k, v, 0.5, shared, bq, bk)
    o_b, l_b = core.attention_blocksparse(q, k, v, 0.5, np.broadcast_to(shared, (H, 4, 5)), bq, bk)
    np.testing.assert_array_equal(o_s, o_b)
    np.testing.assert_array_equal(l_s, l_b)
    # the per-head masks really differ, and so do the results
    assert not np.array_equal(per_head[0], per_head[1])


def test_empty_rows_and_bad_arguments():
    q, k, v = _rand(17, 1, 1, 12, 2)
    m = np.ones((3, 2), dtype=np.uint8)
    m[1] = 0  # rows 4..7 keep no key
    o, lse = core.attention_blocksparse(q, k, v, 1.0, m, 4, 6)
    assert np.all(o[0, 0, 4:8] == 0.0) and np.all(np.isneginf(lse[0, 0, 4:8]))
    assert np.all(np.isfinite(lse[0, 0, :4])) and np.all(np.isfinite(lse[0, 0, 8:]))
    o0, l0 = core.attention_blocksparse(q, k, v, 1.0, np.zeros((3, 2)), 4, 6)
    assert np.all(o0 == 0.0) and np.all(np.isneginf(l0))
    with pytest.raises(ValueError):
        core.attention_blocksparse(q, k, v, 1.0, np.ones((2, 2)), 4, 6)  # wrong number of query blocks
    with pytest.raises(ValueError):
        core.attention_blocksparse(q, k, v, 1.0, m, 0, 6)
    with pytest.raises(RuntimeError):
        core.attention_blocksparse(q, k, v, 1.0, m, 4, 6, window_left=-2)
