"""Throughput of the attention forward (or backward) pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--pass fwd|bwd]
                    [--splits S] [--window-left L --window-right R]
                    [--block-density P [--block-size S]] [--no-cpu-baseline]
    python bench.py --cpu-variant [--workload NAME] [--heads K] [--threads T]

A step is one fa_fwd call over the whole workload (every query row of every
head), with q, k, v already resident in device memory. The default workload is
B=1, H=32, N=8192, d=128, non-causal, fp16. Prints one JSON line.

--splits S times fa_fwd_splitkv with S key splits (0: the library's heuristic) instead of
fa_fwd (with a window: fa_fwd_splitkv_masked; with a block mask: fa_fwd_splitkv_blocksparse);
the roofline then covers both of its kernels (split reduction and merge).

--window-left L / --window-right R time fa_fwd_masked (with --pass bwd: fa_bwd_masked) with that
sliding window (-1 = no limit; the workload's causal flag is then ignored) and price it by the
allowed (row, key) pairs: 4 d flops each (10 d for the backward).

--block-density P times fa_fwd_blocksparse (with --pass bwd: fa_bwd_blocksparse) with a seeded
random block mask (blocks of --block-size S rows and keys, default 128; each block kept with
probability P, the diagonal always), shared by all heads, the workload's causal flag ignored, and
prices it by the allowed (row, key) pairs: 4 d flops each (10 d for the backward).

--cpu-variant times the host-CPU entry point fa_fwd_cpu instead (no GPU needed) on the first K
heads of the workload (default 4), in TFLOP/s of the same flop convention.

--pass bwd times one fa_bwd call instead (dq, dk, dv from q, k, v, o, lse and a
seeded dout, all resident), priced by the conventional backward count of 2.5x
the forward flops (the five products dP = dO V^T, dV = P^T dO, dQ = dS K,
dK = dS^T Q and the recomputed S = Q K^T); the kernels run two more (S and dP
once in each of the two kernels). The roofline object then covers the whole
call (both kernels).

Algorithmic work per launch: 4*B*H*N^2*d flops (the two products QK^T and PV;
halved when causal), i.e. 1.0995e12 for the default workload. The roofline
object prices it against the dense fp16/bf16 matrix-core peak of MI355X
(256 CUs x 2.4 GHz x 4096 flop/clk = 2516.6 TFLOP/s). ``traffic`` is the
device-memory bytes per launch measured with rocprofv3 counters (FETCH_SIZE +
WRITE_SIZE, scaled by the factor a plain copy kernel of known size reads),
taken from the committed summary in profiles/ when it was measured on the
current kernel source, else null.

cpu_baseline: the fp64 CPU oracle (test infrastructure) timed on this host on a
bounded sample of the same workload (the 1024 seeded query rows per head the
parity test checks), converted to TFLOP/s with the same flop convention.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

PEAK_MFMA_F16_TFLOPS = 2516.6  # 256 CU * 2.4 GHz * 4096 flop/clk/CU, dense fp16/bf16
KERNEL_NAME = "fa_fwd_kernel"
HEADLINE_METRIC = "fwd attention TFLOP/s and % MFMA peak at B1 H32 N8192 d128 (fp16)"


def kernel_sha() -> str:
    from exact_tiled_softmax_fa_amd.rocprof_harness import kernel_sha as sha
    return sha()


def measured_traffic(workload_name: str):
    """Bytes per launch from the committed counter summary, if it matches this kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{KERNEL_NAME}_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha256") != kernel_sha():
        return None
    return rec.get("bytes_per_launch")


def _window_keys(i, N, window):
    """Allowed keys of each row i under a (back, ahead) window (-1 = no limit)."""
    import numpy as np
    lo = np.maximum(0, i - window[0]) if window[0] >= 0 else np.zeros_like(i)
    hi = np.minimum(N, i + window[1] + 1) if window[1] >= 0 else np.full_like(i, N)
    return np.maximum(hi - lo, 0)


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


CPU_SAMPLE_ROWS = 3072  # query rows per head the CPU baseline times (about 10 s of the oracle)


def cpu_baseline(w, window=None, blocks=None):
    """The fp64 oracle on CPU_SAMPLE_ROWS seeded rows per head (every row of the small workloads),
    in the GPU line's unit: conventional TFLOP/s, or 4 d flops per allowed pair under a window (the
    masked oracle) or a block mask (the block-sparse oracle; blocks = (block size, mask))."""
    import numpy as np
    from oracle import core

    q, k, v = workloads.make_inputs(w)
    rows = workloads.sample_rows(w, CPU_SAMPLE_ROWS) if w.rows_per_head is not None else None
    if rows is None:
        rows = np.tile(np.arange(w.N, dtype=np.int64), (w.B * w.H, 1))
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    t0 = time.perf_counter()
    if window is not None:
        core.attention_masked(qd, kd, vd, w.scale, window[0], window[1], None, rows)
        what = f"masked oracle, window {window[0]}/{window[1]}"
    elif blocks is not None:
        core.attention_blocksparse(qd, kd, vd, w.scale, blocks[1], blocks[0], blocks[0], rows=rows)
        what = f"block-sparse oracle, {blocks[0]}x{blocks[0]} blocks"
    else:
        core.attention(qd, kd, vd, w.scale, w.causal, rows)
        what = "fp64 three-pass"
    dt = time.perf_counter() - t0
    if window is not None:
        conv = 4.0 * w.d * float(_window_keys(rows, w.N, window).sum())
    elif blocks is not None:
        bs, m = blocks
        kb_keys = np.minimum(w.N, (np.arange(m.shape[1]) + 1) * bs) - np.arange(m.shape[1]) * bs
        conv = 4.0 * w.d * float((np.asarray(m)[rows // bs] * kb_keys).sum())
    else:
        keys = (rows + 1).sum() if w.causal else rows.size * w.N
        flops = 4.0 * w.d * float(keys)
        # the conventional count halves the causal pair count; scale the sample the same way
        conv = flops * (w.flops() / (4.0 * w.d * (w.B * w.H * w.N * (w.N + 1) / 2 if w.causal
                                                   else w.B * w.H * w.N * w.N)))
    full = w.flops() if window is None and blocks is None else None
    return {
        "value": conv / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": core.threads(),
        "cpu": cpu_model(),
        "kind": "oracle",
        "sample": f"{rows.shape[1]} seeded query rows per head x {rows.shape[0]} heads of {w.name} "
                  f"({rows.size} rows, {dt:.2f} s, {what})",
        "rows_per_s": round(rows.size / dt, 1),
        # the whole workload at the sample's rate (plain attention only)
        "extrapolated_full_s": round(full / (conv / dt), 1) if full else None,
    }


def cpu_baseline_bwd(w, window=None, blocks=None):
    """The fp64 backward oracle on one head of the workload (1024 sampled rows of dq and 1024
    sampled keys of dk, dv when the workload samples rows, else everything), in conventional
    backward TFLOP/s: 10 * d flops per (row, key) pair of the parts it computes (allowed pairs
    under a window or a block mask, with the masked or block-sparse backward oracle; blocks =
    (block size, mask))."""
    import numpy as np
    from oracle import core

    q, k, v = workloads.make_inputs(w)
    dout = workloads.make_dout(w)
    head = lambda t: t.reshape(w.B * w.H, w.N, w.d)[:1].double().numpy()  # noqa: E731
    rows, keys = workloads.sample_rows(w), workloads.sample_keys(w)
    rows = None if rows is None else rows[:1]
    keys = None if keys is None else keys[:1]
    t0 = time.perf_counter()
    one = lambda t: head(t).reshape(1, 1, w.N, w.d)  # noqa: E731
    if window is not None:
        core.attention_backward_masked(one(q), one(k), one(v), one(dout), w.scale, window[0], window[1],
                                       rows=rows, keys=keys)
        pairs = float(_window_keys(np.arange(w.N), w.N, window).sum())
    elif blocks is not None:
        bs, m = blocks
        core.attention_backward_blocksparse(one(q), one(k), one(v), one(dout), w.scale, m, bs, bs, rows=rows,
                                            keys=keys)
        pairs = float(workloads.block_mask_pairs(m, w.N, bs, bs))
    else:
        core.attention_backward(head(q), head(k), head(v), head(dout), w.scale, w.causal, rows=rows, keys=keys)
        pairs = w.N * (w.N + 1) / 2 if w.causal else float(w.N) * w.N
    dt = time.perf_counter() - t0
    # every row's statistics cost a full pass; dq and dk/dv are computed for the sampled part only
    frac = 1.0 if rows is None else (rows.shape[1] + keys.shape[1]) / (2.0 * w.N)
    flops = 10.0 * w.d * pairs * (0.4 + 0.6 * frac)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": core.threads(),
        "cpu": cpu_model(),
        "kind": "oracle",
        "sample": f"one head of {w.name}: every row's softmax statistics and D, dq of "
                  f"{'all' if rows is None else rows.shape[1]} rows, dk and dv of "
                  f"{'all' if keys is None else keys.shape[1]} keys ({dt:.2f} s, fp64 chain rule"
                  + (f", window {window[0]}/{window[1]})" if window is not None else
                     f", {blocks[0]}x{blocks[0]} block mask)" if blocks is not None else ")"),
    }


def cpu_variant(w, heads, threads, steps):
    """fa_fwd_cpu on the first `heads` (b, h) heads of the workload; one JSON line."""
    import os
    import exact_tiled_softmax_fa_amd as fa

    q, k, v = workloads.make_inputs(w)
    nh = min(heads, w.B * w.H)
    q, k, v = (t.reshape(w.B * w.H, w.N, w.d)[:nh].reshape(1, nh, w.N, w.d).contiguous() for t in (q, k, v))
    fa.forward_cpu(q[:, :1, :256].contiguous(), k[:, :1, :256].contiguous(), v[:, :1, :256].contiguous(),
                   causal=w.causal, scale=w.scale, num_threads=threads)  # warm-up
    t0 = time.perf_counter()
    for _ in range(steps):
        fa.forward_cpu(q, k, v, causal=w.causal, scale=w.scale, num_threads=threads)
    dt = (time.perf_counter() - t0) / steps
    flops = 4.0 * nh * w.N * w.N * w.d / (2 if w.causal else 1)
    cores = threads if threads > 0 else len(os.sched_getaffinity(0))
    print(json.dumps({
        "metric": f"fwd attention TFLOP/s on the host CPU, tiled online softmax ({w.name}, {nh} heads)",
        "value": round(flops / dt / 1e12, 4), "unit": "TFLOP/s", "n_gpus": 0, "steps": steps,
        "ms_per_step": round(dt * 1e3, 2), "higher_is_better": True, "dtype": w.dtype, "data": "synthetic",
        "cores": cores, "config": {"workload": w.name, "heads": nh, "N": w.N, "d": w.d, "causal": w.causal},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=workloads.HEADLINE.name, choices=sorted(workloads.BY_NAME))
    ap.add_argument("--pass", dest="which", default="fwd", choices=["fwd", "bwd"],
                    help="time the forward pass (default) or the backward pass")
    ap.add_argument("--splits", type=int, default=None,
                    help="run the forward pass as split-KV with this many splits (0: heuristic)")
    ap.add_argument("--window-left", type=int, default=None, help="sliding window: keys back (-1 = all)")
    ap.add_argument("--window-right", type=int, default=None, help="sliding window: keys ahead (-1 = all)")
    ap.add_argument("--block-density", type=float, default=None, help="block-sparse: fraction of blocks kept")
    ap.add_argument("--block-size", type=int, default=128, help="block-sparse: rows and keys per block")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--no-steady-state", action="store_true",
                    help="skip the steady-state figure (profiled runs: only the warm-up and timed steps)")
    ap.add_argument("--cpu-variant", action="store_true", help="time fa_fwd_cpu on host cores instead")
    ap.add_argument("--heads", type=int, default=4, help="--cpu-variant: heads of the workload to run")
    ap.add_argument("--threads", type=int, default=0, help="--cpu-variant: worker threads (0: all)")
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="before timing, run 3 plain device copies of this many MiB (a known-size "
                         "reference for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the forward pass shards over heads with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    if args.cpu_variant:
        cpu_variant(workloads.BY_NAME[args.workload], args.heads, args.threads, max(1, min(args.steps, 3)))
        return

    import torch
    import exact_tiled_softmax_fa_amd as fa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w = workloads.BY_NAME[args.workload]
    host_inputs = workloads.make_inputs(w)
    # provenance of the synthetic inputs: torch version (it draws them) and a digest of each tensor
    inputs_record = {"torch": torch.__version__, "seed": w.seed,
                     "sha256": {name: hashlib.sha256(t.contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()[:16]
                                for name, t in zip(("q", "k", "v"), host_inputs)}}
    q, k, v = (t.cuda() for t in host_inputs)
    del host_inputs
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")

    if args.copy_ref_mib > 0:
        src = torch.empty(args.copy_ref_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step():
        fa.forward(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)

    splits = None
    if args.splits is not None and args.which == "fwd":
        splits = args.splits or fa.splitkv_heuristic(w.B, w.H, w.N, w.d, w.causal)
        ws = torch.empty(max(1, fa.splitkv_workspace_size(w.B, w.H, w.N, w.d, splits)), dtype=torch.uint8,
                         device="cuda")

        def step():  # noqa: F811
            fa.forward(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, num_splits=splits, workspace=ws)

    window = None
    if args.window_left is not None or args.window_right is not None:
        window = (-1 if args.window_left is None else args.window_left,
                  -1 if args.window_right is None else args.window_right)

        if splits is not None:  # the masked split-KV forward
            def step():  # noqa: F811
                fa.forward_masked(q, k, v, window[0], window[1], None, scale=w.scale, out=o, lse=lse,
                                  num_splits=splits, workspace=ws)
        else:
            def step():  # noqa: F811
                fa.forward_masked(q, k, v, window[0], window[1], None, scale=w.scale, out=o, lse=lse)

    blocks = None
    if args.block_density is not None:
        bmask = workloads.make_block_mask(w, args.block_size, args.block_density)
        blocks = (args.block_size, args.block_density, workloads.block_mask_pairs(bmask, w.N, args.block_size,
                                                                                   args.block_size))
        bmask_dev = torch.from_numpy(bmask).cuda()

        if splits is not None:  # the block-sparse split-KV forward
            def step():  # noqa: F811
                fa.forward_blocksparse(q, k, v, bmask_dev, args.block_size, args.block_size, scale=w.scale, out=o,
                                       lse=lse, num_splits=splits, workspace=ws)
        else:
            def step():  # noqa: F811
                fa.forward_blocksparse(q, k, v, bmask_dev, args.block_size, args.block_size, scale=w.scale, out=o,
                                       lse=lse)

    if args.which == "bwd":
        step()
        dout = workloads.make_dout(w).cuda()
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        delta = torch.empty_like(lse)

        def step():  # noqa: F811
            fa.backward(q, k, v, o, lse, dout, causal=w.causal, scale=w.scale, dq=dq, dk=dk, dv=dv, delta=delta)

        if window is not None:
            def step():  # noqa: F811
                fa.backward_masked(q, k, v, o, lse, dout, window[0], window[1], None, scale=w.scale, dq=dq, dk=dk,
                                   dv=dv, delta=delta)
        if blocks is not None:
            def step():  # noqa: F811
                fa.backward_blocksparse(q, k, v, o, lse, dout, bmask_dev, args.block_size, args.block_size,
                                        scale=w.scale, dq=dq, dk=dk, dv=dv, delta=delta)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    # one event between consecutive steps, on the stream the kernels run on
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = ev[0].elapsed_time(ev[-1]) / args.steps  # average launch duration on the kernel's stream
    in_order = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    per_step = sorted(in_order)

    # Reported alongside, never in place of the line above: the same step once the clock has
    # settled. Leaving idle, the chip first clocks high, then its power limit pulls the clock down
    # and lets it recover over some tens of milliseconds (the cycles per launch stay constant; the
    # rocprof summaries give the clock of each timed dispatch), so the K steps after W warm-up
    # steps can run slower than the same steps later on.
    steady_ms = t_steady = None
    if not args.no_steady_state:
        settle_s = 0.3
        t1 = time.perf_counter()
        while time.perf_counter() - t1 < settle_s:
            for _ in range(5):
                step()
            torch.cuda.synchronize()
        ev2 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        t_steady = time.perf_counter() - t0  # seconds from the start of the timed steps
        ev2[0].record(stream)
        for _ in range(args.steps):
            step()
        ev2[1].record(stream)
        torch.cuda.synchronize()
        steady_ms = ev2[0].elapsed_time(ev2[1]) / args.steps

    flops = w.flops() * (2.5 if args.which == "bwd" else 1.0)
    if window is not None:
        import numpy as np
        flops = (4.0 * w.d * w.B * w.H * float(_window_keys(np.arange(w.N), w.N, window).sum())
                 * (2.5 if args.which == "bwd" else 1.0))
    if blocks is not None:
        flops = 4.0 * w.d * w.B * w.H * float(blocks[2]) * (2.5 if args.which == "bwd" else 1.0)
    value = flops / (wall / args.steps) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    out = {
        "metric": (HEADLINE_METRIC if (w.name == workloads.HEADLINE.name and args.which == "fwd" and splits is None
                                       and window is None and blocks is None)
                   else f"{args.which} attention TFLOP/s ({w.name}"
                        + (f", split-KV {splits}" if splits is not None else "")
                        + (f", window {window[0]}/{window[1]}" if window is not None else "")
                        + (f", block-sparse {blocks[0]}x{blocks[0]} blocks, density {blocks[1]}" if blocks else "")
                        + ")"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "pct_mfma_peak": round(100.0 * value / PEAK_MFMA_F16_TFLOPS, 2),
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "num_splits": splits, "window": window,
                   "block_sparse": ({"block": blocks[0], "density": blocks[1], "allowed_pairs_per_head": blocks[2]}
                                    if blocks else None),
                   "global_batch": w.B, "seq_len": w.N, "parallelism": "none"},
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_MFMA_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_MFMA_F16_TFLOPS, 4),
            "traffic": (measured_traffic(w.name) if args.which == "fwd" and splits is None and window is None
                        and blocks is None else None),
            "kernel": ("fa_bwd_dq_kernel + fa_bwd_dkdv_kernel" + (" (masked)" if window is not None else
                                                                  " (block-sparse)" if blocks is not None else "")
                       if args.which == "bwd" else
                       "fa_fwd_kernel (masked)" if window is not None else
                       "fa_fwd_kernel (block-sparse)" if blocks is not None else
                       "fa_fwd_kernel (split) + fa_merge_kernel" if splits is not None else KERNEL_NAME),
            "kernel_ms": round(kernel_ms, 4),
            "kernel_ms_median": round(per_step[len(per_step) // 2], 4),
            "kernel_ms_min": round(per_step[0], 4),
            "kernel_ms_first_last": [round(in_order[0], 4), round(in_order[-1], 4)],
        },
        "steady_state": None if steady_ms is None else {
            "value": round(flops / (steady_ms * 1e-3) / 1e12, 2),
            "pct_mfma_peak": round(100.0 * flops / (steady_ms * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 2),
            "kernel_ms": round(steady_ms, 4),
            "steps": args.steps,
            "after_s": round(t_steady, 2),
            "note": "the same steps after the timed ones and another 0.3 s of them (clock settled); "
                    "context for value, not the value",
        },
        "inputs": inputs_record,
    }
    if not args.no_cpu_baseline:
        if args.which == "fwd":
            out["cpu_baseline"] = cpu_baseline(w, window, (args.block_size, bmask) if blocks else None)
        else:
            out["cpu_baseline"] = cpu_baseline_bwd(w, window, (args.block_size, bmask) if blocks else None)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
