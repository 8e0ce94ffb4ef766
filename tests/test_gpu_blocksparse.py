"""GPU parity of fa_fwd_blocksparse (a mask over blocks of the score matrix) against the fp64 oracle.

The oracle (``core.attention_blocksparse``) is pinned in tests/test_oracle_blocksparse_pins.py;
the tolerances are the forward's. Rows with no allowed key must come back as o = 0 exactly and
lse = -inf. Masks are seeded random bytes (with the densities named in each case), shared by all
heads, given per head, or per (batch, head); block sizes are the multiples of 64 the kernel takes.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import core
from _compare import check_lse, check_o

pytestmark = pytest.mark.gpu


def _mask(seed, shape, p):
    return (np.random.default_rng(seed).random(shape) < p).astype(np.uint8)


def _run(q, k, v, m, bq, bk, wl=-1, wr=-1, seqlens=None, scale=None):
    import exact_tiled_softmax_fa_amd as fa
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    o, lse = fa.forward_blocksparse(q.cuda(), k.cuda(), v.cuda(), torch.from_numpy(m).cuda(), bq, bk, wl, wr, sl,
                                    scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def _compare(o_gpu, lse_gpu, q, k, v, m, bq, bk, scale, dtype, wl=-1, wr=-1, seqlens=None, rows=None):
    B, H, N, d = q.shape
    o_ref, lse_ref = core.attention_blocksparse(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale, m,
                                                bq, bk, wl, wr, seqlens, rows)
    if rows is not None:
        BH = B * H
        o_gpu = np.stack([o_gpu.reshape(BH, N, d)[i, rows[i]] for i in range(BH)])
        lse_gpu = np.stack([lse_gpu.reshape(BH, N)[i, rows[i]] for i in range(BH)])
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), empty), "rows without keys must have lse = -inf"
    assert np.all(o_gpu[empty] == 0.0), "rows without keys must have o = 0"
    ok_o, rep = check_o(o_gpu, o_ref, dtype)
    ok_l, err_l = check_lse(lse_gpu[~empty], lse_ref[~empty]) if (~empty).any() else (True, 0.0)
    print(f"[blocks] bq={bq} bk={bk} wl={wl} wr={wr}: O max-abs {rep['max_abs']:.3e}, lse {err_l:.3e}, "
          f"empty rows {int(empty.sum())}", flush=True)
    assert ok_o, rep
    assert ok_l, err_l


SHAPES = [(1000, 64, "bf16"), (700, 128, "f16"), (129, 128, "bf16"), (2047, 128, "f16")]
BLOCKS = [(64, 64), (128, 64), (64, 192), (256, 128), (384, 256)]


@pytest.mark.parametrize("bq,bk", BLOCKS)
@pytest.mark.parametrize("N,d,dt", SHAPES)
def test_random_shared_masks(N, d, dt, bq, bk):
    q, k, v = workloads.custom_inputs(1, 3, N, d, dt, 1200 + N + bq + bk)
    scale = float(np.float32(1 / np.sqrt(d)))
    m = _mask(N + bq * 7 + bk, (-(-N // bq), -(-N // bk)), 0.4)
    o, lse = _run(q, k, v, m, bq, bk, scale=scale)
    _compare(o, lse, q, k, v, m, bq, bk, scale, dt)


@pytest.mark.parametrize("form", ["head", "batch_head"])
@pytest.mark.parametrize("d,dt", [(64, "f16"), (128, "bf16")])
def test_per_head_masks(form, d, dt):
    B, H, N, bq, bk = 2, 3, 900, 128, 64
    q, k, v = workloads.custom_inputs(B, H, N, d, dt, 1300 + d)
    scale = float(np.float32(1 / np.sqrt(d)))
    shape = (H, 8, 15) if form == "head" else (B, H, 8, 15)
    m = _mask(1301 + d, shape, 0.35)
    o, lse = _run(q, k, v, m, bq, bk, scale=scale)
    _compare(o, lse, q, k, v, m, bq, bk, scale, dt)


@pytest.mark.parametrize("wl,wr,seqlens", [(-1, 0, None), (300, 0, None), (100, 100, None), (-1, -1, [900, 517]),
                                           (-1, 0, [0, 900]), (250, 40, [640, 333])])
def test_with_windows_and_key_lengths(wl, wr, seqlens):
    B, H, N, d, bq, bk = 2, 2, 900, 128, 64, 128
    q, k, v = workloads.custom_inputs(B, H, N, d, "f16", 1400 + max(wl, 0))
    scale = float(np.float32(1 / np.sqrt(d)))
    m = _mask(1401 + max(wr, 0), (-(-N // bq), -(-N // bk)), 0.5)
    o, lse = _run(q, k, v, m, bq, bk, wl, wr, seqlens, scale)
    _compare(o, lse, q, k, v, m, bq, bk, scale, "f16", wl, wr, seqlens)


def test_empty_rows_and_an_empty_mask():
    N, d = 600, 64
    q, k, v = workloads.custom_inputs(1, 2, N, d, "bf16", 1500)
    m = np.ones((10, 5), dtype=np.uint8)
    m[2] = 0   # rows 128 .. 191 keep no key
    m[7] = 0   # rows 448 .. 511
    o, lse = _run(q, k, v, m, 64, 128)
    _compare(o, lse, q, k, v, m, 64, 128, 0.125, "bf16")
    z = np.zeros((10, 5), dtype=np.uint8)
    o, lse = _run(q, k, v, z, 64, 128)
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))


def test_all_ones_agrees_with_fa_fwd():
    import exact_tiled_softmax_fa_amd as fa
    q, k, v = (t.cuda() for t in workloads.custom_inputs(2, 3, 1500, 128, "bf16", 1600))
    ones = torch.ones((24, 12), dtype=torch.uint8, device="cuda")
    for causal in (False, True):
        o_f, l_f = fa.forward(q, k, v, causal=causal)
        o_b, l_b = fa.forward_blocksparse(q, k, v, ones, 64, 128, -1, 0 if causal else -1)
        torch.cuda.synchronize()
        assert (o_f.float() - o_b.float()).abs().max().item() <= 1e-2
        assert (l_f - l_b).abs().max().item() <= 1e-4


def test_block_sparse_on_the_headline_shape():
    w = workloads.HEADLINE
    q, k, v = workloads.make_inputs(w)
    m = _mask(1700, (w.N // 128, w.N // 128), 0.3)
    np.fill_diagonal(m, 1)
    o, lse = _run(q, k, v, m, 128, 128, scale=w.scale)
    _compare(o, lse, q, k, v, m, 128, 128, w.scale, w.dtype, rows=workloads.sample_rows(w))
