"""GPU parity of the backward pass (fa_bwd through the C ABI) against the fp64 backward oracle.

The oracle (``core.attention_backward``) is the chain rule through the definition, pinned by 50-digit
finite differences (tests/test_oracle_bwd_pins.py). Inputs: each workload's seeded q, k, v and a
seeded upstream gradient dout (``workloads.make_dout``); the GPU forward supplies o and lse, as a
training step would.

Tolerance (no stated bound exists for gradients; this one follows from the arithmetic): every
gradient element is a sum of products one of whose factors (p for dv, dS for dk and dq) is rounded
to the storage type before the matrix product, with unit roundoff u = 2^-11 (f16) or 2^-8 (bf16),
and the result is rounded once more on output. Relative to the head's largest gradient magnitude
that gives errors of order u, so the rule is, per head and tensor,
    |g_gpu - g_ref| <= 4 u max(max|g_ref|, 1e-3 max|dv_ref|) + ulp(g_ref) / 2.
(The floor, tied to dv, which is never degenerate, covers tensors whose exact value is 0: with one
key, dk = 0 exactly, and the GPU returns the fp32 rounding residue of dP - D.)
delta (dout . o, fp32, computed from the stored o) gets |err| <= 4 u max|delta_ref| as well.

Large workloads: the GPU runs the full problem; the oracle checks a seeded subset of heads
(``sample_heads``) and, within them, 1024 sampled rows of dq and 1024 sampled keys of dk and dv.
The sum rules sum_j dk_j = 0 and sum_j dv_j = sum_i dout_i, which hold at any size, are checked on
every head of the GPU result.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import core
from _compare import ulp

pytestmark = pytest.mark.gpu

U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
CANARY = 12345.0
PAD = 4096
# heads the oracle recomputes for each workload (all of them for the small ones)
HEADS = {"B1-H1-N256-d64-f16": None, "B4-H16-N2047-d64-bf16": None, "B1-H32-N8192-d128-f16": 2,
         "B2-H16-N8192-d128-bf16-causal": 2, "B1-H8-N32768-d128-bf16-causal-qk4": 1}


def _guarded(shape, dtype):
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * PAD,), CANARY, dtype=dtype, device="cuda")
    buf[PAD:PAD + n] = float("nan")
    return buf, buf[PAD:PAD + n].view(*shape)


def _intact(buf, n):
    return bool((buf[:PAD] == CANARY).all().item() and (buf[PAD + n:] == CANARY).all().item())


def run_backward(q, k, v, dout, causal, scale):
    """GPU forward then backward; returns float64 numpy arrays (dq, dk, dv, delta) [B,H,N,(d)]."""
    import exact_tiled_softmax_fa_amd as fa
    B, H, N, d = q.shape
    qc, kc, vc, dc = (t.cuda() for t in (q, k, v, dout))
    o, lse = fa.forward(qc, kc, vc, causal=causal, scale=scale)
    bufs = [_guarded((B, H, N, d), q.dtype) for _ in range(3)] + [_guarded((B, H, N), torch.float32)]
    dq, dk, dv, delta = (b[1] for b in bufs)
    fa.backward(qc, kc, vc, o, lse, dc, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv, delta=delta)
    torch.cuda.synchronize()
    for (buf, t), name in zip(bufs, ("dq", "dk", "dv", "delta")):
        assert _intact(buf, t.numel()), f"write outside {name}"
    return tuple(t.float().cpu().double().numpy() for t in (dq, dk, dv, delta))


def check_grad(name, g_gpu, g_ref, dtype, dv_ref):
    """Per-head rule of the module docstring; g arrays are [G, R, d], dv_ref the head's dv."""
    g_gpu = np.asarray(g_gpu, dtype=np.float64)
    g_ref = np.asarray(g_ref, dtype=np.float64)
    assert g_gpu.shape == g_ref.shape, (name, g_gpu.shape, g_ref.shape)
    assert np.isfinite(g_gpu).all(), f"{name}: non-finite values"
    G = g_ref.shape[0]
    floor = 1e-3 * np.abs(np.asarray(dv_ref)).reshape(G, -1).max(axis=1)
    scale = np.maximum(np.abs(g_ref).reshape(G, -1).max(axis=1), floor)[:, None, None]
    err = np.abs(g_gpu - g_ref)
    bound = 4 * U[dtype] * scale + 0.5 * ulp(g_ref, dtype)
    rel = float((err / np.maximum(scale, 1e-300)).max())
    print(f"[bwd] {name}: max |err| / max|ref| = {rel:.3e} (rule {4 * U[dtype]:.3e} + ulp/2), "
          f"max|ref| {float(scale.max()):.3e}", flush=True)
    assert np.all(err <= bound), f"{name}: {int(np.sum(err > bound))} elements over the bound; worst rel {rel:.3e}"


def _select(a, heads, idx, BH, N):
    """a: [B,H,N,...] -> [len(heads), R, ...] rows idx[g] of head heads[g] (idx None: all rows)."""
    a = a.reshape(BH, N, *a.shape[3:])[heads]
    if idx is None:
        return a
    return np.stack([a[g, idx[g]] for g in range(len(heads))])


@pytest.mark.parametrize("name", [w.name for w in workloads.WORKLOADS])
def test_backward_parity(name):
    w = workloads.BY_NAME[name]
    print(f"\n[bwd] {w.name} seed={w.seed} shape=({w.B},{w.H},{w.N},{w.d}) causal={w.causal}", flush=True)
    q, k, v = workloads.make_inputs(w)
    dout = workloads.make_dout(w)
    dq, dk, dv, delta = run_backward(q, k, v, dout, w.causal, w.scale)
    BH, N, d = w.B * w.H, w.N, w.d
    nh = HEADS[w.name]
    heads = workloads.sample_heads(w, nh) if nh is not None else np.arange(BH)
    rows = workloads.sample_rows(w)
    keys = workloads.sample_keys(w)
    rows = None if rows is None else rows[heads]
    keys = None if keys is None else keys[heads]
    flat = lambda t: t.reshape(BH, N, d)[heads].double().numpy()  # noqa: E731
    ref = core.attention_backward(flat(q), flat(k), flat(v), flat(dout), w.scale, w.causal, rows=rows, keys=keys)
    dq_ref, dk_ref, dv_ref, _, delta_ref = ref
    check_grad("dq", _select(dq, heads, rows, BH, N), dq_ref, w.dtype, dv_ref)
    check_grad("dk", _select(dk, heads, keys, BH, N), dk_ref, w.dtype, dv_ref)
    check_grad("dv", _select(dv, heads, keys, BH, N), dv_ref, w.dtype, dv_ref)
    d_gpu = delta.reshape(BH, N)[heads]
    d_err = np.abs(d_gpu - delta_ref).max() / np.abs(delta_ref).max()
    print(f"[bwd] delta: max |err| / max|ref| = {d_err:.3e}", flush=True)
    assert d_err <= 4 * U[w.dtype]
    # sum rules on every head of the full GPU result (fp64 sums of the stored values)
    dk_h = dk.reshape(BH, N, d)
    dv_h = dv.reshape(BH, N, d)
    do_h = dout.reshape(BH, N, d).double().numpy()
    k_sum = np.abs(dk_h.sum(axis=1)).max() / np.abs(dk_h).sum(axis=1).max()
    v_sum = np.abs(dv_h.sum(axis=1) - do_h.sum(axis=1)).max() / np.abs(do_h).sum(axis=1).max()
    print(f"[bwd] sum rules: |sum dk| / sum|dk| = {k_sum:.3e}, |sum dv - sum dout| / sum|dout| = {v_sum:.3e}",
          flush=True)
    assert k_sum <= U[w.dtype] and v_sum <= U[w.dtype]


# (300 and 600: odd counts of 128-key and of 256-row tiles, where a paired causal workgroup takes the
# middle tile alone)
TAIL_CASES = [(N, d, causal, dt) for N in (1, 17, 64, 100, 129, 255, 300, 600) for d in (64, 128)
              for causal in (False, True) for dt in ("f16", "bf16")]


@pytest.mark.parametrize("N,d,causal,dt", TAIL_CASES)
def test_backward_tails(N, d, causal, dt):
    seed = 100 + N + d + (7 if causal else 0) + (3 if dt == "bf16" else 0)
    q, k, v = workloads.custom_inputs(1, 2, N, d, dt, seed)
    g = torch.Generator().manual_seed(seed + 2000)
    dout = torch.randn((1, 2, N, d), generator=g).to(q.dtype)
    scale = float(np.float32(1 / np.sqrt(d)))
    dq, dk, dv, delta = run_backward(q, k, v, dout, causal, scale)
    ref = core.attention_backward(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                  dout.double().numpy(), scale, causal)
    for name, a, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        check_grad(f"{name} N={N} d={d} causal={causal} {dt}", a.reshape(2, N, d), r, dt, ref[2])
    assert np.abs(delta.reshape(2, N) - ref[4]).max() <= 4 * U[dt] * np.abs(ref[4]).max() + 1e-6


def test_backward_is_deterministic():
    import exact_tiled_softmax_fa_amd as fa
    q, k, v = (t.cuda() for t in workloads.custom_inputs(1, 4, 1000, 128, "bf16", 77))
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(78)).to(q.dtype).cuda()
    o, lse = fa.forward(q, k, v, causal=True)
    first = fa.backward(q, k, v, o, lse, dout, causal=True)
    for _ in range(5):
        again = fa.backward(q, k, v, o, lse, dout, causal=True)
        for a, b in zip(first, again):
            assert torch.equal(a, b)


def test_backward_zero_keys_closed_form():
    """K = 0: every row weights its keys uniformly, so dv_j = sum_i dout_i / N (non-causal) and dq = 0."""
    import exact_tiled_softmax_fa_amd as fa
    q, _, v = (t.cuda() for t in workloads.custom_inputs(1, 2, 200, 64, "f16", 90))
    k = torch.zeros_like(q)
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(91)).to(q.dtype).cuda()
    o, lse = fa.forward(q, k, v)
    dq, dk, dv = fa.backward(q, k, v, o, lse, dout)
    assert torch.count_nonzero(dq).item() == 0
    expect = dout.double().mean(dim=2, keepdim=True).expand_as(dv)
    err = (dv.double() - expect).abs().max().item()
    amax = expect.abs().max().item()
    assert err <= 4 * U["f16"] * amax + 0.5 * float(ulp(amax, "f16")), err
