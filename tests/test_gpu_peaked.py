"""GPU parity on peaked logits: q and k drawn with standard deviation 2 or 3, so a row's logits
have a standard deviation of 4 or 9 and a few keys carry nearly all of its weight.

This is the regime where rounding the probabilities to the operand type of the second product
matters most: a bf16 probability is off by up to 2^-8 of itself, and when two or three keys share
a row's weight, those errors move O by up to about 2^-8 |v_i - v_j|. The bf16 kernels keep the
exact running maximum, so the largest weight is exactly 1 ("transformer math: flash attention
math", aicassindra.com, "The block-wise update, and the full algorithm"); the f16 kernels (11
significant bits) keep the lazy reference.

Every forward entry point is compared elementwise with the fp64 oracle under the rule of
``_compare.py``, on fixed seeds. The first case is a shape and seed on which the lazy bf16
reference measured 1.02e-2, above the bound.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import core
from _compare import check_lse, check_o

pytestmark = pytest.mark.gpu


def _host(o, lse):
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def _check(tag, o_gpu, lse_gpu, o_ref, lse_ref, dtype):
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), empty), "rows without keys must have lse = -inf"
    assert np.all(o_gpu[empty] == 0.0), "rows without keys must have o = 0"
    ok_o, rep = check_o(o_gpu, o_ref, dtype)
    ok_l, err_l = check_lse(lse_gpu[~empty], lse_ref[~empty]) if (~empty).any() else (True, 0.0)
    print(f"[peaked] {tag}: O max-abs {rep['max_abs']:.3e} (over tol {rep['n_over_tol']} of {rep['n']}), "
          f"lse max-abs {err_l:.3e}", flush=True)
    assert ok_o, rep
    assert ok_l, err_l


def test_bf16_case_the_lazy_reference_failed():
    import exact_tiled_softmax_fa_amd as fa
    B, H, N, d, seed = 2, 1, 2214, 128, 1048243725
    print(f"\n[peaked] fa_fwd B{B} H{H} N{N} d{d} bf16 sigma 3 seed {seed}", flush=True)
    q, k, v = workloads.custom_inputs(B, H, N, d, "bf16", seed, sigma_qk=3.0)
    scale = float(np.float32(1 / np.sqrt(d)))
    o, lse = _host(*fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=False, scale=scale))
    o_ref, lse_ref = core.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale, False)
    _check("fa_fwd case", o, lse, o_ref, lse_ref, "bf16")


ENTRIES = ["plain", "causal", "masked", "splitkv", "blocksparse", "splitkv_masked", "splitkv_blocksparse"]


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("sigma", [2.0, 3.0])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_peaked_logits_every_entry_point(entry, sigma, dt, d):
    import exact_tiled_softmax_fa_amd as fa
    B, H, N = 2, 2, 1437  # several 256-row query tiles, a ragged 64-key tail
    seed = 5100 + 97 * ENTRIES.index(entry) + 13 * int(sigma) + (7 if dt == "bf16" else 0) + d
    print(f"\n[peaked] {entry} B{B} H{H} N{N} d{d} {dt} sigma {sigma} seed {seed}", flush=True)
    q, k, v = workloads.custom_inputs(B, H, N, d, dt, seed, sigma_qk=sigma)
    scale = float(np.float32(1 / np.sqrt(d)))
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    wl, wr, seqlens = 300, 40, [N, 1000]
    bq, bk = 128, 64
    m = (np.random.default_rng(seed).random((-(-N // bq), -(-N // bk))) < 0.5).astype(np.uint8)
    np.fill_diagonal(m[:, ::2], 1)
    sl = torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    if entry in ("plain", "causal"):
        causal = entry == "causal"
        res = fa.forward(qc, kc, vc, causal=causal, scale=scale)
        ref = core.attention(qd, kd, vd, scale, causal)
    elif entry == "splitkv":
        res = fa.forward(qc, kc, vc, causal=False, scale=scale, num_splits=3)
        ref = core.attention(qd, kd, vd, scale, False)
    elif entry in ("masked", "splitkv_masked"):
        kw = {"num_splits": 3} if entry == "splitkv_masked" else {}
        res = fa.forward_masked(qc, kc, vc, wl, wr, sl, scale=scale, **kw)
        ref = core.attention_masked(qd, kd, vd, scale, wl, wr, seqlens)
    else:
        kw = {"num_splits": 3} if entry == "splitkv_blocksparse" else {}
        res = fa.forward_blocksparse(qc, kc, vc, torch.from_numpy(m).cuda(), bq, bk, scale=scale, **kw)
        ref = core.attention_blocksparse(qd, kd, vd, scale, m, bq, bk)
    o, lse = _host(*res)
    _check(f"{entry} {dt} d{d} sigma {sigma}", o, lse, np.asarray(ref[0]), np.asarray(ref[1]), dt)
