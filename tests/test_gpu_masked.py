"""GPU parity of fa_fwd_masked (sliding windows, key padding) against the masked fp64 oracle.

The oracle (``core.attention_masked``) is pinned in tests/test_oracle_mask_pins.py; tolerances are
the forward's. Rows with no allowed key must come back as o = 0 exactly and lse = -inf.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import core
from _compare import check_lse, check_o

pytestmark = pytest.mark.gpu


def _run(q, k, v, wl, wr, seqlens, scale):
    import exact_tiled_softmax_fa_amd as fa
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    o, lse = fa.forward_masked(q.cuda(), k.cuda(), v.cuda(), wl, wr, sl, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def _compare(o_gpu, lse_gpu, q, k, v, wl, wr, seqlens, scale, dtype, rows=None):
    B, H, N, d = q.shape
    o_ref, lse_ref = core.attention_masked(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale,
                                           wl, wr, seqlens, rows)
    if rows is not None:
        BH = B * H
        o_gpu = np.stack([o_gpu.reshape(BH, N, d)[i, rows[i]] for i in range(BH)])
        lse_gpu = np.stack([lse_gpu.reshape(BH, N)[i, rows[i]] for i in range(BH)])
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), empty), "rows without keys must have lse = -inf"
    assert np.all(o_gpu[empty] == 0.0), "rows without keys must have o = 0"
    ok_o, rep = check_o(o_gpu, o_ref, dtype)
    ok_l, err_l = check_lse(lse_gpu[~empty], lse_ref[~empty]) if (~empty).any() else (True, 0.0)
    print(f"[mask] wl={wl} wr={wr} seqlens={seqlens}: O max-abs {rep['max_abs']:.3e}, lse {err_l:.3e}, "
          f"empty rows {int(empty.sum())}", flush=True)
    assert ok_o, rep
    assert ok_l, err_l


WINDOWS = [(0, 0), (31, 0), (100, 0), (257, 0), (63, 63), (-1, 5), (200, -1), (1, 300)]


@pytest.mark.parametrize("wl,wr", WINDOWS)
@pytest.mark.parametrize("N,d,dt", [(700, 64, "f16"), (1000, 128, "bf16"), (129, 128, "f16")])
def test_sliding_windows(wl, wr, N, d, dt):
    q, k, v = workloads.custom_inputs(1, 2, N, d, dt, 800 + N + max(wl, 0))
    scale = float(np.float32(1 / np.sqrt(d)))
    o, lse = _run(q, k, v, wl, wr, None, scale)
    _compare(o, lse, q, k, v, wl, wr, None, scale, dt)


@pytest.mark.parametrize("wl,wr,seqlens", [(-1, -1, [700, 513, 1]), (-1, 0, [64, 700, 300]),
                                           (128, 0, [0, 650, 699]), (50, 10, [700, 0, 256])])
@pytest.mark.parametrize("d,dt", [(64, "bf16"), (128, "f16")])
def test_key_padding(wl, wr, seqlens, d, dt):
    q, k, v = workloads.custom_inputs(3, 2, 700, d, dt, 900 + d)
    scale = float(np.float32(1 / np.sqrt(d)))
    o, lse = _run(q, k, v, wl, wr, seqlens, scale)
    _compare(o, lse, q, k, v, wl, wr, seqlens, scale, dt)


def test_local_attention_on_the_headline_shape():
    w = workloads.HEADLINE
    q, k, v = workloads.make_inputs(w)
    o, lse = _run(q, k, v, 1023, 0, None, w.scale)
    _compare(o, lse, q, k, v, 1023, 0, None, w.scale, w.dtype, workloads.sample_rows(w))


def test_general_kernel_agrees_with_the_causal_one():
    import exact_tiled_softmax_fa_amd as fa
    q, k, v = (t.cuda() for t in workloads.custom_inputs(2, 3, 1500, 128, "bf16", 950))
    o_c, l_c = fa.forward(q, k, v, causal=True)
    full = torch.full((2,), 1500, dtype=torch.int32, device="cuda")  # forces the general kernel
    o_m, l_m = fa.forward_masked(q, k, v, -1, 0, full)
    torch.cuda.synchronize()
    assert (o_c.float() - o_m.float()).abs().max().item() <= 1e-2
    assert (l_c - l_m).abs().max().item() <= 1e-4


@pytest.mark.parametrize("wl,wr", [(2047, 0), (2048, 0), (1023, 1024), (1024, 1024), (0, 2047)])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_windows_around_the_four_wave_limit(wl, wr, dt):
    # at d = 128, windows of up to 2048 keys run 128-row workgroups, wider ones 256-row workgroups
    q, k, v = workloads.custom_inputs(1, 2, 3000, 128, dt, 960 + wl + wr)
    scale = float(np.float32(1 / np.sqrt(128)))
    o, lse = _run(q, k, v, wl, wr, None, scale)
    _compare(o, lse, q, k, v, wl, wr, None, scale, dt)


def test_narrow_window_on_the_headline_shape():
    w = workloads.HEADLINE
    q, k, v = workloads.make_inputs(w)
    o, lse = _run(q, k, v, 255, 0, None, w.scale)
    _compare(o, lse, q, k, v, 255, 0, None, w.scale, w.dtype, workloads.sample_rows(w))


@pytest.mark.parametrize("d", [64, 128])
def test_windows_of_n_minus_one_keys_are_no_limit(d):
    # a window of N - 1 keys back (or ahead) excludes no key: the call is plain or causal fa_fwd
    import exact_tiled_softmax_fa_amd as fa
    N = 777
    q, k, v = (t.cuda() for t in workloads.custom_inputs(1, 2, N, d, "f16", 970 + d))
    for (wl, wr), causal in (((N - 1, 0), True), ((N - 1, N - 1), False), ((-1, N - 1), False)):
        o_m, l_m = fa.forward_masked(q, k, v, wl, wr)
        o_f, l_f = fa.forward(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o_m, o_f) and torch.equal(l_m, l_f), (wl, wr)
    o, lse = _run(q.cpu(), k.cpu(), v.cpu(), N - 2, 0, None, None)  # one key short of causal
    _compare(o, lse, q.cpu(), k.cpu(), v.cpu(), N - 2, 0, None, float(np.float32(1 / np.sqrt(d))), "f16")
