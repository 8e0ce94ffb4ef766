"""GPU parity of fa_bwd_masked (gradients under a sliding window and key lengths) against the fp64
masked backward oracle.

The oracle (``core.attention_backward_masked``) is pinned in tests/test_oracle_bwd_mask_pins.py. The
GPU forward under the same mask (fa_fwd_masked) supplies o and lse, as a training step would. The
tolerance rule is the backward's (tests/test_gpu_backward.py). Rows with no allowed key must give
dq = 0 exactly, keys no row allows dk = dv = 0 exactly, and no output may be written outside its
tensor.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import core
from test_gpu_backward import U, _guarded, _intact, check_grad

pytestmark = pytest.mark.gpu


def _run(q, k, v, dout, wl, wr, seqlens, scale):
    import exact_tiled_softmax_fa_amd as fa
    B, H, N, d = q.shape
    qc, kc, vc, dc = (t.cuda() for t in (q, k, v, dout))
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    o, lse = fa.forward_masked(qc, kc, vc, wl, wr, sl, scale=scale)
    bufs = [_guarded((B, H, N, d), q.dtype) for _ in range(3)] + [_guarded((B, H, N), torch.float32)]
    dq, dk, dv, delta = (b[1] for b in bufs)
    fa.backward_masked(qc, kc, vc, o, lse, dc, wl, wr, sl, scale=scale, dq=dq, dk=dk, dv=dv, delta=delta)
    torch.cuda.synchronize()
    for (buf, t), name in zip(bufs, ("dq", "dk", "dv", "delta")):
        assert _intact(buf, t.numel()), f"write outside {name}"
    return tuple(t.float().cpu().double().numpy() for t in (dq, dk, dv, delta))


def _compare(got, q, k, v, dout, wl, wr, seqlens, scale, dt, heads=None):
    B, H, N, d = q.shape
    G = B * H
    dq, dk, dv, delta = (a.reshape(G, N, -1) if a.ndim == 4 else a.reshape(G, N) for a in got)
    arrs = [t.double().numpy() for t in (q, k, v, dout)]
    rq, rk, rv, rl, rd = core.attention_backward_masked(*arrs, scale, wl, wr, seqlens)
    if heads is not None:
        dq, dk, dv, delta, rq, rk, rv, rl, rd = (a[heads] for a in (dq, dk, dv, delta, rq, rk, rv, rl, rd))
    empty_rows = np.isneginf(rl)
    assert np.all(dq[empty_rows] == 0.0), "rows without keys must get dq = 0"
    dead_keys = (np.abs(rk).max(axis=-1) == 0) & (np.abs(rv).max(axis=-1) == 0)
    assert np.all(dk[dead_keys] == 0.0) and np.all(dv[dead_keys] == 0.0), "keys no row allows: dk = dv = 0"
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        check_grad(name, g, r, dt, rv)
    err_d = np.abs(delta - rd).max()
    assert err_d <= 4 * U[dt] * max(np.abs(rd).max(), 1e-30) + 1e-7, err_d


WINDOWS = [(0, 0), (31, 0), (100, 0), (63, 63), (-1, 5), (200, -1), (1, 300)]


@pytest.mark.parametrize("wl,wr", WINDOWS)
@pytest.mark.parametrize("N,d,dt", [(700, 64, "f16"), (1000, 128, "bf16"), (129, 128, "f16")])
def test_sliding_windows(wl, wr, N, d, dt):
    q, k, v = workloads.custom_inputs(1, 2, N, d, dt, 1900 + N + max(wl, 0))
    dout = workloads.custom_inputs(1, 2, N, d, dt, 1950 + N)[0]
    scale = float(np.float32(1 / np.sqrt(d)))
    got = _run(q, k, v, dout, wl, wr, None, scale)
    _compare(got, q, k, v, dout, wl, wr, None, scale, dt)


@pytest.mark.parametrize("wl,wr,seqlens", [(-1, -1, [700, 513, 1]), (-1, 0, [64, 700, 300]),
                                           (128, 0, [0, 650, 699]), (50, 10, [700, 0, 256])])
@pytest.mark.parametrize("d,dt", [(64, "bf16"), (128, "f16")])
def test_key_padding(wl, wr, seqlens, d, dt):
    q, k, v = workloads.custom_inputs(3, 2, 700, d, dt, 2000 + d)
    dout = workloads.custom_inputs(3, 2, 700, d, dt, 2001 + d)[0]
    scale = float(np.float32(1 / np.sqrt(d)))
    got = _run(q, k, v, dout, wl, wr, seqlens, scale)
    _compare(got, q, k, v, dout, wl, wr, seqlens, scale, dt)


def test_local_window_on_the_headline_shape():
    w = workloads.HEADLINE
    q, k, v = workloads.make_inputs(w)
    dout = workloads.make_dout(w)
    heads = workloads.sample_heads(w, 2)
    got = _run(q, k, v, dout, 1023, 0, None, w.scale)
    # the oracle on the sampled heads only (every row and key of them)
    B, H, N, d = q.shape
    nh = len(heads)

    def sel(a):
        return a.reshape(B * H, N, *a.shape[3:])[heads].reshape(1, nh, N, *a.shape[3:])

    _compare(tuple(sel(a) for a in got), sel(q), sel(k), sel(v), sel(dout), 1023, 0, None, w.scale, w.dtype)


def test_trivial_masks_run_fa_bwd():
    import exact_tiled_softmax_fa_amd as fa
    q, k, v, dout = (t.cuda() for t in workloads.custom_inputs(2, 2, 600, 64, "f16", 2100) +
                     (workloads.custom_inputs(2, 2, 600, 64, "f16", 2101)[0],))
    for wr, causal in ((-1, False), (0, True)):
        o, lse = fa.forward(q, k, v, causal=causal)
        a = fa.backward(q, k, v, o, lse, dout, causal=causal)
        b = fa.backward_masked(q, k, v, o, lse, dout, -1, wr)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y)


def test_general_kernel_agrees_with_the_causal_one():
    import exact_tiled_softmax_fa_amd as fa
    q, k, v, dout = (t.cuda() for t in workloads.custom_inputs(2, 3, 1500, 128, "bf16", 2200) +
                     (workloads.custom_inputs(2, 3, 1500, 128, "bf16", 2201)[0],))
    o, lse = fa.forward(q, k, v, causal=True)
    a = fa.backward(q, k, v, o, lse, dout, causal=True)
    full = torch.full((2,), 1500, dtype=torch.int32, device="cuda")  # forces the general kernels
    b = fa.backward_masked(q, k, v, o, lse, dout, -1, 0, full)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        scale = x.float().abs().max().item()
        assert (x.float() - y.float()).abs().max().item() <= 4 * U["bf16"] * scale


@pytest.mark.parametrize("wl,wr", [(2047, 0), (2048, 0), (1023, 1024), (1024, 1024)])
def test_windows_around_the_four_wave_limit(wl, wr):
    # at d = 128 the dq kernel runs 128-row workgroups for windows of up to 2048 keys, 256-row ones
    # beyond
    N, d, dt = 2600, 128, "bf16"
    q, k, v = workloads.custom_inputs(1, 1, N, d, dt, 2200 + wl + wr)
    dout = workloads.custom_inputs(1, 1, N, d, dt, 2201 + wl + wr)[0]
    scale = float(np.float32(1 / np.sqrt(d)))
    got = _run(q, k, v, dout, wl, wr, None, scale)
    _compare(got, q, k, v, dout, wl, wr, None, scale, dt)


@pytest.mark.parametrize("d", [64, 128])
def test_windows_of_n_minus_one_keys_are_no_limit(d):
    # a window of N - 1 keys back (or ahead) excludes no key: the call is plain or causal fa_bwd
    import exact_tiled_softmax_fa_amd as fa
    N = 777
    q, k, v, dout = (t.cuda() for t in workloads.custom_inputs(1, 2, N, d, "f16", 2300 + d) +
                     (workloads.custom_inputs(1, 2, N, d, "f16", 2301 + d)[0],))
    for (wl, wr), causal in (((N - 1, 0), True), ((N - 1, N - 1), False)):
        o, lse = fa.forward(q, k, v, causal=causal)
        a = fa.backward(q, k, v, o, lse, dout, causal=causal)
        b = fa.backward_masked(q, k, v, o, lse, dout, wl, wr)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y), (wl, wr)
