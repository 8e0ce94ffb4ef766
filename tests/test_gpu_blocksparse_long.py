"""GPU parity of the block-sparse forward and backward beyond 65536 keys, against the fp64 oracle.

One work list of a workgroup holds 1024 tiles of 64 (65536 keys or query rows); longer sequences
run the kernels that build and walk the list a chunk of 1024 candidate tiles at a time, the
online state carrying over between chunks. These cases put more than 1024 candidate tiles in a
workgroup's range (no window), so every workgroup walks two chunks, with ragged tails, and
masks chosen so that some query blocks keep keys only in the first chunk, some only in the
second, some in both and some none. Outputs are compared on sampled rows (and, for dk and dv,
sampled keys) including the first and last rows and those around the chunk boundary; the
oracles and tolerances are those of tests/test_gpu_blocksparse.py and
tests/test_gpu_backward_blocksparse.py.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import core
from _compare import check_lse, check_o
from test_gpu_backward import U, check_grad

pytestmark = pytest.mark.gpu

CHUNK_KEYS = 64 * 1024  # keys (or query rows) one work list covers


def _sample(N, count, seed, extra=()):
    rng = np.random.default_rng(seed)
    fixed = [0, N - 1, CHUNK_KEYS - 1, CHUNK_KEYS, CHUNK_KEYS - 64, CHUNK_KEYS + 63, *extra]
    pick = rng.choice(N, size=count, replace=False)
    return np.unique(np.concatenate([np.array([r for r in fixed if 0 <= r < N], dtype=np.int64), pick]))


def _forward(q, k, v, m, bq, bk, wl=-1, wr=-1, seqlens=None, scale=None):
    import exact_tiled_softmax_fa_amd as fa
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    o, lse = fa.forward_blocksparse(q.cuda(), k.cuda(), v.cuda(), torch.from_numpy(m).cuda(), bq, bk, wl, wr, sl,
                                    scale=scale)
    torch.cuda.synchronize()
    return o, lse


def _check_forward(o, lse, q, k, v, m, bq, bk, scale, dt, rows, wl=-1, wr=-1, seqlens=None):
    B, H, N, d = q.shape
    G = B * H
    ridx = np.stack([rows] * G)
    o_ref, lse_ref = core.attention_blocksparse(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale,
                                                m, bq, bk, wl, wr, seqlens, ridx)
    o_gpu = o.float().cpu().double().numpy().reshape(G, N, d)[:, rows]
    lse_gpu = lse.cpu().double().numpy().reshape(G, N)[:, rows]
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), empty), "rows without keys must have lse = -inf"
    assert np.all(o_gpu[empty] == 0.0), "rows without keys must have o = 0"
    ok_o, rep = check_o(o_gpu, o_ref, dt)
    ok_l, err_l = check_lse(lse_gpu[~empty], lse_ref[~empty]) if (~empty).any() else (True, 0.0)
    print(f"[blocks long] N={N} d={d} {dt} bq={bq} bk={bk}: {len(rows)} rows/head, O max-abs "
          f"{rep['max_abs']:.3e}, lse {err_l:.3e}, empty rows {int(empty.sum())}", flush=True)
    assert ok_o, rep
    assert ok_l, err_l
    return empty


def _random_mask(seed, shape, p, bq, bk):
    """Seeded random bytes with the diagonal blocks kept (every row keeps its own key)."""
    m = (np.random.default_rng(seed).random(shape) < p).astype(np.uint8)
    nq, nk = shape[-2:]
    for i in range(nq):
        m[..., i, min((i * bq) // bk, nk - 1)] = 1
    return m


@pytest.mark.parametrize("d,dt", [(64, "bf16"), (128, "f16")])
def test_random_per_head_masks_past_one_list(d, dt):
    N, bq, bk = CHUNK_KEYS + 64 * 3 + 29, 64, 64
    q, k, v = workloads.custom_inputs(1, 2, N, d, dt, 4100 + d)
    scale = float(np.float32(1 / np.sqrt(d)))
    m = _random_mask(4101 + d, (2, -(-N // bq), -(-N // bk)), 0.02, bq, bk)
    o, lse = _forward(q, k, v, m, bq, bk, scale=scale)
    _check_forward(o, lse, q, k, v, m, bq, bk, scale, dt, _sample(N, 40, 4102 + d))


def test_keys_only_in_one_chunk():
    # query block r (128 rows) keeps: r % 4 == 0 -> only the two key blocks past 65536 (second
    # chunk); 1 -> only key blocks 0 and 255 (first chunk, its first and last); 2 -> both; 3 -> none
    N, d, dt, bq, bk = 66000, 128, "f16", 128, 256
    q, k, v = workloads.custom_inputs(1, 1, N, d, dt, 4200)
    nq, nk = -(-N // bq), -(-N // bk)
    m = np.zeros((nq, nk), dtype=np.uint8)
    for r in range(nq):
        if r % 4 == 0:
            m[r, 256:] = 1
        elif r % 4 == 1:
            m[r, [0, 255]] = 1
        elif r % 4 == 2:
            m[r, [3, 100, 255, 256, nk - 1]] = 1
    scale = float(np.float32(1 / np.sqrt(d)))
    o, lse = _forward(q, k, v, m, bq, bk, scale=scale)
    rows = _sample(N, 48, 4201, extra=[128 * r + e for r in (0, 1, 2, 3, 511, 512, 513, 514, 515) for e in (0, 127)])
    empty = _check_forward(o, lse, q, k, v, m, bq, bk, scale, dt, rows)
    assert empty.any() and not empty.all()


def test_key_lengths_and_per_batch_masks_past_one_list():
    N, d, dt, bq, bk = CHUNK_KEYS + 300, 64, "bf16", 192, 128
    q, k, v = workloads.custom_inputs(2, 1, N, d, dt, 4300)
    m = _random_mask(4301, (2, 1, -(-N // bq), -(-N // bk)), 0.03, bq, bk)
    seqlens = [N, CHUNK_KEYS + 37]
    o, lse = _forward(q, k, v, m, bq, bk, seqlens=seqlens, scale=0.125)
    _check_forward(o, lse, q, k, v, m, bq, bk, 0.125, dt, _sample(N, 40, 4302), seqlens=seqlens)


@pytest.mark.parametrize("d,dt", [(64, "f16"), (128, "bf16")])
def test_backward_past_one_list(d, dt):
    import exact_tiled_softmax_fa_amd as fa
    N, bq, bk = CHUNK_KEYS + 64 + 17, 64, 128
    q, k, v = workloads.custom_inputs(1, 1, N, d, dt, 4400 + d)
    dout = workloads.custom_inputs(1, 1, N, d, dt, 4401 + d)[0]
    scale = float(np.float32(1 / np.sqrt(d)))
    m = _random_mask(4402 + d, (-(-N // bq), -(-N // bk)), 0.02, bq, bk)
    m[7] = 0  # query rows 448 .. 511 keep no key
    o, lse = _forward(q, k, v, m, bq, bk, scale=scale)
    mc = torch.from_numpy(m).cuda()
    dq, dk, dv, delta = fa.backward_blocksparse(q.cuda(), k.cuda(), v.cuda(), o, lse, dout.cuda(), mc, bq, bk,
                                                scale=scale, return_delta=True)
    torch.cuda.synchronize()
    rows = _sample(N, 40, 4403 + d, extra=[448, 511])
    keys = _sample(N, 40, 4404 + d)
    arrs = [t.double().numpy() for t in (q, k, v, dout)]
    rq, rk, rv, rl, rd = core.attention_backward_blocksparse(*arrs, scale, m, bq, bk, rows=rows[None, :],
                                                             keys=keys[None, :])
    g = lambda t: t.float().cpu().double().numpy().reshape(1, N, -1)  # noqa: E731
    dq_s, dk_s, dv_s = g(dq)[:, rows], g(dk)[:, keys], g(dv)[:, keys]
    assert np.all(dq_s[:, np.isin(rows, np.arange(448, 512))] == 0.0), "rows without keys must get dq = 0"
    for name, got, ref in (("dq", dq_s, rq), ("dk", dk_s, rk), ("dv", dv_s, rv)):
        check_grad(name, got, ref, dt, rv)
    dl = delta.cpu().double().numpy().reshape(1, N)
    err_d = np.abs(dl - rd).max()
    assert err_d <= 4 * U[dt] * max(np.abs(rd).max(), 1e-30) + 1e-7, err_d
