"""rocprofv3 harness: kernel time, matrix-core utilisation, clock, instruction mix and device-memory
traffic, all measured on the same timed dispatches.

    python -m exact_tiled_softmax_fa_amd.rocprof_harness [--workload NAME] [--pass fwd|bwd]
                                                         [--steps K] [--warmup W]
                                                         [--out DIR] [--summary-dir DIR] [--parse-only]

--pass fwd (default) profiles fa_fwd's kernel; --pass bwd profiles the two kernels of fa_bwd
(fa_bwd_dq_kernel, fa_bwd_dkdv_kernel), each summarised on its own; --splits S (with --pass fwd)
profiles fa_fwd_splitkv's split kernel and its merge kernel; --block-density P [--block-size S]
(with --pass fwd) profiles fa_fwd_blocksparse on bench.py's seeded block mask, priced by the
allowed (row, key) pairs.

Every pass runs the same command, ``bench.py --steps K --warmup W`` (default K = 20, W = 5: the
command a default benchmark line is measured with), as a child process (this process never touches
the GPU, so the profiler's preload stays in its own process):

1. ``--kernel-trace --stats``: per-dispatch kernel durations, no counters.
2. ``--kernel-trace --pmc FETCH_SIZE`` and 3. ``--kernel-trace --pmc WRITE_SIZE``, one counter per
   pass, with a plain 256 MiB device copy run first (``bench.py --copy-ref-mib 256``). The copy's
   known size calibrates both counters (bytes read and written by a copy of known size / counter
   value), and the same factors scale the kernel's counts.
4. ``--kernel-trace --pmc SQ_INSTS_VALU_MFMA_MOPS_{F16,BF16} SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES
   GRBM_GUI_ACTIVE``: matrix-core work and busy cycles against elapsed cycles.
5. ``--kernel-trace --pmc SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_SALU SQ_INSTS_LDS
   SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_COEXEC_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY GRBM_GUI_ACTIVE``:
   the instruction mix and where the waves' cycles go.

In every pass the timed dispatches are the kernel's dispatches W+1 .. W+K in dispatch-id order: the
same K calls the benchmark times, after its W warm-up calls (the profiled command skips the
benchmark's steady-state block). Each counter is averaged over those
dispatches of its own pass, and the clock is each dispatch's GUI-active cycles per XCD over that
same dispatch's duration in the same pass (a counter pass serialises dispatches, so its durations
are not the benchmark's; they only pair cycles with time). It then writes a Markdown summary
(``<summary-dir>/fa_fwd_kernel_<workload>.md``) and ``traffic_fa_fwd_kernel_<workload>.json``. The
JSON holds the bytes per launch and the SHA-256 of the kernel source it was measured on;
``bench.py`` reports the traffic only while that hash matches. Reported figures:
- the per-dispatch durations of the trace pass and their mean over the timed dispatches;
- MFMA busy fraction = busy cycles / SIMDs / (GUI-active cycles / XCDs);
- the clock of the timed dispatches, and the dense MFMA peak scaled to it;
- vector, matrix, scalar and LDS instructions per launch, and the fractions of wave cycles spent
  issuing vector work, waiting for issue and waiting on counters or barriers;
- device-memory bytes per launch and the achieved GB/s (bytes / mean kernel time);
- the ratio of measured to unavoidable bytes (Q, K, V read once; O, lse written once).
"""
import argparse
import csv
import hashlib
import json
import os
import shlex
import statistics
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
# each pass's kernel sources: its own file and the device helpers it includes
KERNEL_SRCS = {
    "fwd": [os.path.join(HERE, "csrc", "fa_fwd.hip"), os.path.join(HERE, "csrc", "fa_device.h")],
    "bwd": [os.path.join(HERE, "csrc", "fa_bwd.hip"), os.path.join(HERE, "csrc", "fa_device.h")],
}
N_SIMD = 1024   # MI355X: 256 CUs x 4 SIMDs
N_XCD = 8
COPY_MIB = 256
PEAK_TFLOPS = 2516.6  # MI355X dense fp16/bf16 matrix-core peak
PEAK_CLOCK_GHZ = 2.4  # the clock that peak is quoted at


def kernel_sha(which: str = "fwd") -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS[which]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


MIX_COUNTERS = ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_ACTIVE_INST_VALU",
                "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "GRBM_GUI_ACTIVE"]


def passes(workload: str, out: str, steps: int, warmup: int, which: str = "fwd", splits=None, blocks=None):
    bench = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", workload, "--pass", which,
             "--no-cpu-baseline", "--no-steady-state"]
    if splits is not None:
        bench += ["--splits", str(splits)]
    if blocks is not None:
        bench += ["--block-size", str(blocks[0]), "--block-density", str(blocks[1])]
    timed = bench + ["--steps", str(steps), "--warmup", str(warmup)]
    copy = ["--copy-ref-mib", str(COPY_MIB)]
    dtype_mops = "SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU_MFMA_MOPS_BF16".split()
    kt = ["--kernel-trace"]
    return [
        ("kt", ["--kernel-trace", "--stats"], timed),
        ("fetch", kt + ["--pmc", "FETCH_SIZE"], timed + copy),
        ("write", kt + ["--pmc", "WRITE_SIZE"], timed + copy),
        ("mfma", kt + ["--pmc", *dtype_mops, "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"], timed),
        ("mix", kt + ["--pmc", *MIX_COUNTERS], timed),
    ]


def display_command(cmd: str) -> str:
    """A recorded command as run from the repository root: the interpreter as python3 and the
    benchmark and output paths relative to the root (the absolute ones name one machine's copy)."""
    words = []
    for w in shlex.split(cmd):
        if w == sys.executable or (os.path.isabs(w) and os.path.basename(w).startswith("python")):
            w = "python3"
        elif os.path.isabs(w) and w.endswith("/bench.py"):
            w = "bench.py"
        elif os.path.isabs(w) and os.path.commonpath([w, ROOT]) == ROOT:
            w = os.path.relpath(w, ROOT)
        words.append(w)
    return " ".join(shlex.quote(w) for w in words)


def run(workload: str, out: str, steps: int, warmup: int, timeout: int, which: str = "fwd", splits=None,
        blocks=None) -> list:
    cmds = []
    for name, prof_args, prog in passes(workload, out, steps, warmup, which, splits, blocks):
        cmd = ["rocprofv3", *prof_args, "--output-format", "csv", "-d", os.path.join(out, name), "-o", name,
               "--", *prog]
        cmds.append(display_command(" ".join(shlex.quote(c) for c in cmd)))
        print(f"[rocprof] {name}: {cmds[-1]}", flush=True)
        env = dict(os.environ, TMPDIR=os.environ.get("TMPDIR", "/tmp"))
        res = subprocess.run(cmd, env=env, timeout=timeout)
        if res.returncode != 0:
            raise RuntimeError(f"rocprofv3 pass {name} failed with exit code {res.returncode}")
    return cmds


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(out, name, suffix):
    d = os.path.join(out, name)
    for dirpath, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(dirpath, f)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def _reference_copies(values):
    """The counter values of the reference copies among a run's copy dispatches: the runtime's
    own small copies (a block mask uploaded to the device, say) use the same copy kernel, so
    only dispatches of at least half the largest one's size count."""
    if not values:
        return values
    top = max(values)
    return [v for v in values if v >= 0.5 * top]


def timed_dispatches(rows, kernel: str, steps: int, warmup: int):
    """Dispatch ids of a pass's timed calls of `kernel`: in id order, the `steps` dispatches after its
    first `warmup` ones (the benchmark's warm-up calls come first). Works on kernel-trace and
    counter-collection rows."""
    ids = sorted({int(r["Dispatch_Id"]) for r in rows if kernel in r["Kernel_Name"]})
    return ids[warmup:warmup + steps]


def _durations_ms(out, name):
    """Dispatch id -> duration (ms) from a pass's kernel trace."""
    return {int(r["Dispatch_Id"]): (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
            for r in _rows(_find(out, name, "kernel_trace.csv"))}


def _counter(out, name, counter, kernel, steps=None, warmup=0):
    """Per-dispatch values of `counter` for `kernel` in pass `name`: {dispatch id: value}, restricted
    to the timed dispatches when `steps` is given."""
    rows = [r for r in _rows(_find(out, name, "counter_collection.csv")) if kernel in r["Kernel_Name"]]
    keep = set(timed_dispatches(rows, kernel, steps, warmup)) if steps else None
    vals = {}
    for r in rows:
        if r["Counter_Name"] == counter and (keep is None or int(r["Dispatch_Id"]) in keep):
            vals[int(r["Dispatch_Id"])] = vals.get(int(r["Dispatch_Id"]), 0.0) + float(r["Counter_Value"])
    return vals


def _mean(d):
    return statistics.mean(d.values()) if d else 0.0


def kernels(workload: str, which: str = "fwd", splits=None, blocks=None):
    """(kernel name, matrix-product flops per launch, unavoidable bytes per launch) of a pass.
    Flops: 2 N^2 d per product per head (halved when causal); forward: the two products of the
    conventional count; backward: the products each kernel executes (dq: S, dP, dQ; dkdv: S, dP,
    dV, dK). Unavoidable bytes: every tensor the kernel must read or write, once."""
    sys.path.insert(0, ROOT)
    import workloads

    w = workloads.BY_NAME[workload]
    BH, N, d = w.B * w.H, w.N, w.d
    per_product = 2.0 * BH * N * N * d / (2 if w.causal else 1)
    t = N * d * 2  # one [N, d] tensor of one head
    if which == "fwd" and splits:
        # split reduction: reads q, k, v, writes the partials (fp32 o and two lse per row and split);
        # merge: reads the partials, writes o and lse
        part = splits * BH * N * (d + 2) * 4
        return [("fa_fwd_kernel", 2 * per_product, BH * 3 * t + part),
                ("fa_merge_kernel", 0.0, part + BH * (t + 4 * N))]
    if blocks:
        # the block-sparse kernels: 2 d flops per product and allowed (row, key) pair of bench.py's
        # seeded mask (forward 2 products, dq 3, dkdv 4)
        m = workloads.make_block_mask(w, blocks[0], blocks[1])
        pairs = workloads.block_mask_pairs(m, N, blocks[0], blocks[0])
        if which == "fwd":
            return [("fa_fwd_kernel", 4.0 * d * BH * pairs, BH * (4 * t + 4 * N))]
        return [("fa_bwd_dq_kernel", 6.0 * d * BH * pairs, BH * (6 * t + 8 * N)),
                ("fa_bwd_dkdv_kernel", 8.0 * d * BH * pairs, BH * (6 * t + 8 * N))]
    if which == "fwd":
        return [("fa_fwd_kernel", 2 * per_product, BH * (4 * t + 4 * N))]
    return [("fa_bwd_dq_kernel", 3 * per_product, BH * (6 * t + 8 * N)),   # q k v o dO lse -> dq delta
            ("fa_bwd_dkdv_kernel", 4 * per_product, BH * (6 * t + 8 * N))]  # q k v dO lse delta -> dk dv


def summarize(workload: str, out: str, steps: int, cmds=None, which: str = "fwd", splits=None, blocks=None,
              warmup: int = 0) -> list:
    """One record per kernel of the pass (see ``kernels``)."""
    recs = []
    for kname, flops, unavoidable in kernels(workload, which, splits, blocks):
        trace = _rows(_find(out, "kt", "kernel_trace.csv"))
        dur = _durations_ms(out, "kt")
        all_ids = sorted({int(r["Dispatch_Id"]) for r in trace if kname in r["Kernel_Name"]})
        durs = [dur[i] for i in all_ids]
        timed = [dur[i] for i in timed_dispatches(trace, kname, steps, warmup)]
        ms = statistics.mean(timed)
        fetch_copy = _reference_copies(list(_counter(out, "fetch", "FETCH_SIZE", "copyBuffer").values()))
        write_copy = _reference_copies(list(_counter(out, "write", "WRITE_SIZE", "copyBuffer").values()))
        f_fac = COPY_MIB * 1024.0 / statistics.mean(fetch_copy)
        w_fac = COPY_MIB * 1024.0 / statistics.mean(write_copy)
        fetch_b = _mean(_counter(out, "fetch", "FETCH_SIZE", kname, steps, warmup)) * f_fac * 1024
        write_b = _mean(_counter(out, "write", "WRITE_SIZE", kname, steps, warmup)) * w_fac * 1024
        gui_d = _counter(out, "mfma", "GRBM_GUI_ACTIVE", kname, steps, warmup)
        gui = _mean(gui_d)
        busy = _mean(_counter(out, "mfma", "SQ_VALU_MFMA_BUSY_CYCLES", kname, steps, warmup))
        mops = sum(_mean(_counter(out, "mfma", c, kname, steps, warmup))
                   for c in ("SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_BF16"))
        util = busy / N_SIMD / (gui / N_XCD) if gui else 0.0
        # clock: each timed dispatch's cycles over its own duration, in the same (counter) pass
        dur_mfma = _durations_ms(out, "mfma")
        clocks = [gui_d[i] / N_XCD / (dur_mfma[i] * 1e-3) / 1e9 for i in gui_d if dur_mfma.get(i)]
        mix = {}
        try:
            for c in MIX_COUNTERS:
                mix[c] = _mean(_counter(out, "mix", c, kname, steps, warmup))
        except FileNotFoundError:
            mix = {}
        recs.append({
            "kernel": kname,
            "kernel_sha256": kernel_sha(which),
            "workload": workload,
            "steps": steps,
            "warmup": warmup,
            "kernel_ms_mean_timed": ms,
            "dispatch_ms": durs,
            "bytes_per_launch": fetch_b + write_b,
            "fetch_bytes": fetch_b,
            "write_bytes": write_b,
            "fetch_scale": f_fac,
            "write_scale": w_fac,
            "achieved_gb_per_s": (fetch_b + write_b) / (ms * 1e-3) / 1e9,
            "unavoidable_bytes": unavoidable,
            "traffic_over_unavoidable": (fetch_b + write_b) / unavoidable,
            "mfma_flop_per_launch": mops * 512,
            "mfma_busy_fraction": util,
            "tflops_from_trace": flops / (ms * 1e-3) / 1e12,
            "clock_ghz": statistics.mean(clocks) if clocks else 0.0,
            "instruction_mix": mix,
            "commands": cmds or [],
            "pass": which,
            "splits": splits,
            "blocks": list(blocks) if blocks else None,
        })
    return recs


def variant_tag(splits=None, blocks=None) -> str:
    """File-name suffix of a profiled variant."""
    return (f"_split{splits}" if splits else "") + (f"_blocks{blocks[0]}_p{blocks[1]}" if blocks else "")


def clock_line(rec: dict) -> str:
    """The clock line of a summary: the timed dispatches' GUI-active cycles per XCD over their own
    durations, both from the matrix-core counter pass."""
    ghz = rec["clock_ghz"]
    if rec["mfma_flop_per_launch"] <= 0 or ghz <= 0:
        return "- clock of the timed dispatches: not given (no matrix work or no cycle count)"
    return (f"- clock of the timed dispatches: {ghz:.2f} GHz (cycles and durations of the same dispatches); "
            f"dense MFMA peak at that clock: {PEAK_TFLOPS * ghz / PEAK_CLOCK_GHZ:.0f} TFLOP/s "
            f"(of {PEAK_TFLOPS} at {PEAK_CLOCK_GHZ} GHz)")


def mix_lines(rec: dict) -> list:
    """Instruction mix per launch and the split of wave cycles (from the mix counter pass)."""
    m = rec.get("instruction_mix") or {}
    if not m or not m.get("SQ_INSTS_VALU"):
        return []
    lines = ["## Instruction mix (SQ_INSTS_*, SQ_ACTIVE_INST_VALU, SQ_WAIT_*; per launch)", "",
             f"- vector instructions {m['SQ_INSTS_VALU']:.4g} (of which MFMA {m['SQ_INSTS_MFMA']:.4g}), "
             f"scalar {m['SQ_INSTS_SALU']:.4g}, LDS {m['SQ_INSTS_LDS']:.4g}"]
    gui = m.get("GRBM_GUI_ACTIVE", 0.0)
    if gui:
        simd_cycles = gui / N_XCD * N_SIMD
        lines.append(f"- vector issue busy (incl. MFMA issue) {100 * 4 * m['SQ_ACTIVE_INST_VALU'] / simd_cycles:.1f} % "
                     f"of SIMD cycles; MFMA busy while a vector instruction issued (co-execution) "
                     f"{100 * m['SQ_VALU_MFMA_COEXEC_CYCLES'] / simd_cycles:.1f} %")
        lines.append(f"- wave cycles waiting on counters or barriers {4 * m['SQ_WAIT_ANY'] / simd_cycles:.2f}, "
                     f"waiting to issue {4 * m['SQ_WAIT_INST_ANY'] / simd_cycles:.2f} (wave-cycles per SIMD cycle)")
    lines.append("")
    return lines


def write_summary(rec: dict, summary_dir: str):
    os.makedirs(summary_dir, exist_ok=True)
    name = f"{rec['kernel']}_{rec['workload']}" + variant_tag(rec.get("splits"), rec.get("blocks"))
    lines = [f"# {rec['kernel']} — {rec['workload']}", ""]
    if rec["commands"]:
        lines += ["Made by `python -m exact_tiled_softmax_fa_amd.rocprof_harness --workload "
                  f"{rec['workload']} --pass {rec['pass']}"
                  + (f" --splits {rec['splits']}" if rec.get("splits") else "")
                  + (f" --block-size {rec['blocks'][0]} --block-density {rec['blocks'][1]}" if rec.get("blocks")
                     else "")
                  + f" --steps {rec.get('steps')} --warmup {rec.get('warmup', 0)}"
                  + "` (repository root, on the GPU), which ran:", "", "```",
                  *[display_command(c) for c in rec["commands"]], "```", ""]
    d = rec["dispatch_ms"]
    w0 = rec.get("warmup", 0)
    if len(d) <= 40:
        disp = [f"- dispatches (ms): {', '.join(f'{x:.3f}' for x in d)}"]
    else:  # long warm-ups: their range, then the timed dispatches
        warm = d[:w0]
        disp = [f"- warm-up dispatches 1 .. {w0} (ms): first {warm[0]:.3f}, min {min(warm):.3f}, "
                f"max {max(warm):.3f}, last {warm[-1]:.3f}" if warm else "- no warm-up dispatches",
                f"- timed dispatches (ms): {', '.join(f'{x:.3f}' for x in d[w0:])}"]
    lines += [
        "## Kernel time (rocprofv3 --kernel-trace --stats)", "",
        *disp,
        f"- mean of the timed dispatches ({rec.get('warmup', 0) + 1} .. {rec.get('warmup', 0) + rec.get('steps', len(d))}): **{rec['kernel_ms_mean_timed']:.4f} ms** "
        f"= {rec['tflops_from_trace']:.1f} TFLOP/s (the matrix products this kernel executes)", "",
        "## Device-memory traffic (FETCH_SIZE, WRITE_SIZE; one counter per pass)", "",
        f"- scale factors from a {COPY_MIB} MiB device copy: fetch x{rec['fetch_scale']:.3f}, "
        f"write x{rec['write_scale']:.3f}",
        f"- per launch: {rec['fetch_bytes'] / 2**20:.1f} MiB read + {rec['write_bytes'] / 2**20:.1f} MiB written "
        f"= {rec['bytes_per_launch'] / 2**20:.1f} MiB; unavoidable (each tensor read or written once) "
        f"{rec['unavoidable_bytes'] / 2**20:.1f} MiB; ratio {rec['traffic_over_unavoidable']:.3f}",
        f"- achieved device-memory bandwidth: {rec['achieved_gb_per_s']:.1f} GB/s (of about 8000)", "",
        "## Matrix cores (SQ_INSTS_VALU_MFMA_MOPS_*, SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE)", "",
        f"- MFMA work per launch: {rec['mfma_flop_per_launch']:.4e} flop",
        f"- MFMA busy: **{100 * rec['mfma_busy_fraction']:.1f} %** of elapsed cycles",
        clock_line(rec), "",
    ] + mix_lines(rec)
    with open(os.path.join(summary_dir, name + ".md"), "w") as f:
        f.write("\n".join(lines))
    slim = {k: v for k, v in rec.items() if k != "dispatch_ms"}
    slim["commands"] = [display_command(c) for c in rec["commands"]]
    with open(os.path.join(summary_dir, "traffic_" + name + ".json"), "w") as f:
        json.dump(slim, f, indent=1)
    print("\n".join(lines), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="B1-H32-N8192-d128-f16")
    ap.add_argument("--pass", dest="which", default="fwd", choices=["fwd", "bwd"])
    ap.add_argument("--splits", type=int, default=None, help="profile fa_fwd_splitkv with this many splits")
    ap.add_argument("--block-density", type=float, default=None,
                    help="profile fa_fwd_blocksparse (fa_bwd_blocksparse with --pass bwd) at this density")
    ap.add_argument("--block-size", type=int, default=128, help="block-sparse: rows and keys per block")
    ap.add_argument("--out", default=os.path.join(ROOT, "rocprof_out"))
    ap.add_argument("--summary-dir", default=os.path.join(ROOT, "rocprof_out"))
    # every pass runs the calls of the benchmark command the headline line is measured with
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--timeout", type=int, default=240, help="seconds per rocprofv3 pass")
    ap.add_argument("--parse-only", action="store_true", help="summarise existing outputs under --out")
    args = ap.parse_args()
    blocks = (args.block_size, args.block_density) if args.block_density is not None else None
    tag = f"{args.which}_{args.workload}" + variant_tag(args.splits, blocks)
    out = os.path.join(args.out, tag)
    cmds = None
    if not args.parse_only:
        cmds = run(args.workload, out, args.steps, args.warmup, args.timeout, args.which, args.splits, blocks)
    for rec in summarize(args.workload, out, args.steps, cmds, args.which, args.splits, blocks, args.warmup):
        if args.parse_only:  # keep the commands an earlier summary of the same run recorded
            name = f"{rec['kernel']}_{rec['workload']}" + variant_tag(rec.get("splits"), rec.get("blocks"))
            prev = os.path.join(args.summary_dir, "traffic_" + name + ".json")
            if os.path.exists(prev):
                with open(prev) as f:
                    rec["commands"] = json.load(f).get("commands", [])
        write_summary(rec, args.summary_dir)


if __name__ == "__main__":
    main()
