"""GPU parity of fa_bwd_blocksparse (gradients under a block mask, optionally with a window and key
lengths) against the fp64 oracle.

The oracle (``core.attention_backward_blocksparse``) is pinned in
tests/test_oracle_bwd_blocksparse_pins.py. The GPU forward under the same masks
(fa_fwd_blocksparse) supplies o and lse, as a training step would. The tolerance rule is the
backward's (tests/test_gpu_backward.py). Rows with no allowed key must give dq = 0 exactly, keys
no row allows dk = dv = 0 exactly, and no output may be written outside its tensor. Masks are
seeded random bytes with the densities named in each case; block sizes are the multiples of 64
the kernels take, chosen so that block edges fall inside the kernels' 256-row and 128-key
workgroups as well as on them.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import core
from test_gpu_backward import U, _guarded, _intact, check_grad

pytestmark = pytest.mark.gpu


def _mask(seed, shape, p):
    return (np.random.default_rng(seed).random(shape) < p).astype(np.uint8)


def _run(q, k, v, dout, m, bq, bk, wl=-1, wr=-1, seqlens=None, scale=None):
    import exact_tiled_softmax_fa_amd as fa
    B, H, N, d = q.shape
    qc, kc, vc, dc = (t.cuda() for t in (q, k, v, dout))
    mc = torch.from_numpy(m).cuda()
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    o, lse = fa.forward_blocksparse(qc, kc, vc, mc, bq, bk, wl, wr, sl, scale=scale)
    bufs = [_guarded((B, H, N, d), q.dtype) for _ in range(3)] + [_guarded((B, H, N), torch.float32)]
    dq, dk, dv, delta = (b[1] for b in bufs)
    fa.backward_blocksparse(qc, kc, vc, o, lse, dc, mc, bq, bk, wl, wr, sl, scale=scale, dq=dq, dk=dk, dv=dv,
                            delta=delta)
    torch.cuda.synchronize()
    for (buf, t), name in zip(bufs, ("dq", "dk", "dv", "delta")):
        assert _intact(buf, t.numel()), f"write outside {name}"
    return tuple(t.float().cpu().double().numpy() for t in (dq, dk, dv, delta))


def _compare(got, q, k, v, dout, m, bq, bk, scale, dt, wl=-1, wr=-1, seqlens=None):
    B, H, N, d = q.shape
    G = B * H
    dq, dk, dv, delta = (a.reshape(G, N, -1) if a.ndim == 4 else a.reshape(G, N) for a in got)
    arrs = [t.double().numpy() for t in (q, k, v, dout)]
    rq, rk, rv, rl, rd = core.attention_backward_blocksparse(*arrs, scale, m, bq, bk, wl, wr, seqlens)
    empty_rows = np.isneginf(rl)
    assert np.all(dq[empty_rows] == 0.0), "rows without keys must get dq = 0"
    assert np.all(delta[empty_rows] == 0.0), "rows without keys have o = 0, so D = dout . o = 0"
    dead_keys = (np.abs(rk).max(axis=-1) == 0) & (np.abs(rv).max(axis=-1) == 0)
    assert np.all(dk[dead_keys] == 0.0) and np.all(dv[dead_keys] == 0.0), "keys no row allows: dk = dv = 0"
    print(f"[bwd blocks] bq={bq} bk={bk} wl={wl} wr={wr}: empty rows {int(empty_rows.sum())}, "
          f"dead keys {int(dead_keys.sum())}", flush=True)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        check_grad(name, g, r, dt, rv)
    err_d = np.abs(delta - rd).max()
    assert err_d <= 4 * U[dt] * max(np.abs(rd).max(), 1e-30) + 1e-7, err_d


SHAPES = [(700, 64, "f16"), (1000, 128, "bf16"), (129, 128, "f16")]
BLOCKS = [(64, 64), (128, 64), (64, 192), (256, 128), (384, 320)]


@pytest.mark.parametrize("bq,bk", BLOCKS)
@pytest.mark.parametrize("N,d,dt", SHAPES)
def test_random_shared_masks(N, d, dt, bq, bk):
    q, k, v = workloads.custom_inputs(1, 2, N, d, dt, 2300 + N + bq + bk)
    dout = workloads.custom_inputs(1, 2, N, d, dt, 2301 + N)[0]
    scale = float(np.float32(1 / np.sqrt(d)))
    m = _mask(N + 3 * bq + bk, (-(-N // bq), -(-N // bk)), 0.4)
    got = _run(q, k, v, dout, m, bq, bk, scale=scale)
    _compare(got, q, k, v, dout, m, bq, bk, scale, dt)


@pytest.mark.parametrize("form", ["head", "batch_head"])
@pytest.mark.parametrize("d,dt", [(64, "bf16"), (128, "f16")])
def test_per_head_masks(form, d, dt):
    B, H, N, bq, bk = 2, 3, 900, 128, 64
    q, k, v = workloads.custom_inputs(B, H, N, d, dt, 2400 + d)
    dout = workloads.custom_inputs(B, H, N, d, dt, 2401 + d)[0]
    scale = float(np.float32(1 / np.sqrt(d)))
    shape = (H, 8, 15) if form == "head" else (B, H, 8, 15)
    m = _mask(2402 + d, shape, 0.35)
    got = _run(q, k, v, dout, m, bq, bk, scale=scale)
    _compare(got, q, k, v, dout, m, bq, bk, scale, dt)


@pytest.mark.parametrize("wl,wr,seqlens", [(-1, 0, None), (300, 0, None), (100, 100, None), (-1, -1, [900, 517]),
                                           (-1, 0, [0, 900]), (250, 40, [640, 333])])
def test_with_windows_and_key_lengths(wl, wr, seqlens):
    B, H, N, d, bq, bk = 2, 2, 900, 128, 64, 128
    q, k, v = workloads.custom_inputs(B, H, N, d, "bf16", 2500 + max(wl, 0))
    dout = workloads.custom_inputs(B, H, N, d, "bf16", 2501 + max(wr, 0))[0]
    scale = float(np.float32(1 / np.sqrt(d)))
    m = _mask(2502 + max(wr, 0), (-(-N // bq), -(-N // bk)), 0.5)
    got = _run(q, k, v, dout, m, bq, bk, wl, wr, seqlens, scale)
    _compare(got, q, k, v, dout, m, bq, bk, scale, "bf16", wl, wr, seqlens)


def test_empty_rows_and_an_empty_mask():
    N, d = 600, 64
    q, k, v = workloads.custom_inputs(1, 2, N, d, "f16", 2600)
    dout = workloads.custom_inputs(1, 2, N, d, "f16", 2601)[0]
    m = np.ones((10, 5), dtype=np.uint8)
    m[2] = 0     # rows 128 .. 191 keep no key
    m[:, 3] = 0  # keys 384 .. 511: no row
    got = _run(q, k, v, dout, m, 64, 128)
    _compare(got, q, k, v, dout, m, 64, 128, 0.125, "f16")
    z = np.zeros((10, 5), dtype=np.uint8)
    dq, dk, dv, delta = _run(q, k, v, dout, z, 64, 128)
    assert np.all(dq == 0.0) and np.all(dk == 0.0) and np.all(dv == 0.0) and np.all(delta == 0.0)


def test_all_ones_agrees_with_fa_bwd():
    import exact_tiled_softmax_fa_amd as fa
    q, k, v, dout = (t.cuda() for t in workloads.custom_inputs(2, 3, 1500, 128, "bf16", 2700) +
                     (workloads.custom_inputs(2, 3, 1500, 128, "bf16", 2701)[0],))
    ones = torch.ones((24, 12), dtype=torch.uint8, device="cuda")
    for causal in (False, True):
        o, lse = fa.forward(q, k, v, causal=causal)
        a = fa.backward(q, k, v, o, lse, dout, causal=causal)
        b = fa.backward_blocksparse(q, k, v, o, lse, dout, ones, 64, 128, -1, 0 if causal else -1)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            scale = x.float().abs().max().item()
            assert (x.float() - y.float()).abs().max().item() <= 4 * U["bf16"] * scale


def test_block_sparse_backward_on_the_headline_shape():
    w = workloads.HEADLINE
    q, k, v = workloads.make_inputs(w)
    dout = workloads.make_dout(w)
    m = workloads.make_block_mask(w, 128, 0.25)
    got = _run(q, k, v, dout, m, 128, 128, scale=w.scale)
    # the oracle on two sampled heads (every row and key of them); the mask is shared by all heads
    heads = workloads.sample_heads(w, 2)
    B, H, N, d = q.shape
    nh = len(heads)

    def sel(a):
        return a.reshape(B * H, N, *a.shape[3:])[heads].reshape(1, nh, N, *a.shape[3:])

    _compare(tuple(sel(a) for a in got), sel(q), sel(k), sel(v), sel(dout), m, 128, 128, w.scale, w.dtype)
