"""The rocprof harness's parsing and arithmetic, on synthetic rocprofv3 CSV files (no GPU)."""
import csv
import json
import os

import pytest

from exact_tiled_softmax_fa_amd import rocprof_harness as rh

KERNEL = "void (anonymous namespace)::fa_fwd_kernel<128, false, false>(...)"
COPY = "__amd_rocclr_copyBuffer"
TRACE_FIELDS = ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
PMC_FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
WARM, STEPS = 3, 20


def _write(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _trace(path, durs_ns, first_id=1, copies=0):
    """A kernel trace: `copies` copy dispatches, then the kernel's dispatches of the given durations."""
    t, rows, i = 0, [], first_id
    for _ in range(copies):
        rows.append({"Dispatch_Id": i, "Kernel_Name": COPY, "Start_Timestamp": t, "End_Timestamp": t + 5_000_000})
        t += 5_001_000
        i += 1
    for d in durs_ns:
        rows.append({"Dispatch_Id": i, "Kernel_Name": KERNEL, "Start_Timestamp": t, "End_Timestamp": t + d})
        t += d + 1000
        i += 1
    _write(path, TRACE_FIELDS, rows)


def _pmc(path, values, copy_values=(), first_id=1):
    """Counter rows: per kernel dispatch a dict counter -> value (warm-up dispatches first)."""
    rows, i = [], first_id
    for cv in copy_values:
        rows.append({"Dispatch_Id": i, "Kernel_Name": COPY, "Counter_Name": cv[0], "Counter_Value": cv[1]})
        i += 1
    for per in values:
        for name, v in per.items():
            rows.append({"Dispatch_Id": i, "Kernel_Name": KERNEL, "Counter_Name": name, "Counter_Value": v})
        i += 1
    _write(path, PMC_FIELDS, rows)


@pytest.fixture
def fake_run(tmp_path):
    out = str(tmp_path / "run")
    # WARM warm-up dispatches at 2 ms, STEPS timed ones at 1 ms, then 5 more (not timed) at 3 ms
    durs = [2_000_000] * WARM + [1_000_000] * STEPS + [3_000_000] * 5
    _trace(os.path.join(out, "kt", "h", "kt_kernel_trace.csv"), durs)
    # counter passes: warm-up dispatches carry different values, which must not enter the means
    # the copy reference reads half its size in FETCH_SIZE units and writes its full size
    for name, counter, timed_v, copy_v in (("fetch", "FETCH_SIZE", 100000.0, 131072.0),
                                           ("write", "WRITE_SIZE", 66560.0, 262144.0)):
        _trace(os.path.join(out, name, "h", f"{name}_kernel_trace.csv"), durs, copies=3)
        _pmc(os.path.join(out, name, "h", f"{name}_counter_collection.csv"),
             [{counter: 7.0}] * WARM + [{counter: timed_v}] * STEPS + [{counter: 9.0}] * 5, [(counter, copy_v)] * 3)
    # matrix pass: its dispatches last 1 ms with 2e6 GUI-active cycles per XCD (2 GHz) when timed
    _trace(os.path.join(out, "mfma", "h", "mfma_kernel_trace.csv"), durs)
    _pmc(os.path.join(out, "mfma", "h", "mfma_counter_collection.csv"),
         [{"SQ_INSTS_VALU_MFMA_MOPS_F16": 1.0, "SQ_VALU_MFMA_BUSY_CYCLES": 1.0, "GRBM_GUI_ACTIVE": 8.0}] * WARM +
         [{"SQ_INSTS_VALU_MFMA_MOPS_F16": 2 ** 31, "SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 1e6,
           "GRBM_GUI_ACTIVE": 8 * 2e6}] * STEPS)
    _trace(os.path.join(out, "mix", "h", "mix_kernel_trace.csv"), durs)
    _pmc(os.path.join(out, "mix", "h", "mix_counter_collection.csv"),
         [{c: 1.0 for c in rh.MIX_COUNTERS}] * WARM +
         [{"SQ_INSTS_VALU": 3e8, "SQ_INSTS_MFMA": 6.7e7, "SQ_INSTS_SALU": 3e7, "SQ_INSTS_LDS": 5e7,
           "SQ_ACTIVE_INST_VALU": 0.25 * 2e6 * 1024, "SQ_VALU_MFMA_COEXEC_CYCLES": 0.1 * 2e6 * 1024,
           "SQ_WAIT_ANY": 0.1 * 2e6 * 1024, "SQ_WAIT_INST_ANY": 0.2 * 2e6 * 1024, "GRBM_GUI_ACTIVE": 8 * 2e6}] * STEPS)
    return out


def test_timed_dispatches_are_the_last_steps_by_id():
    rows = [{"Dispatch_Id": str(i), "Kernel_Name": KERNEL if i % 3 else COPY} for i in (9, 1, 4, 2, 5, 7, 8, 10, 11)]
    # kernel dispatches (ids not divisible by 3): 1 2 4 5 7 8 10 11; the last 3 are 8 10 11
    assert rh.timed_dispatches(rows, "fa_fwd_kernel", 3, 2) == [4, 5, 7]
    assert rh.timed_dispatches(rows, "fa_fwd_kernel", 50, 0) == [1, 2, 4, 5, 7, 8, 10, 11]
    assert rh.timed_dispatches(rows, "fa_fwd_kernel", 3, 6) == [10, 11]


def test_counters_average_only_the_timed_dispatches(fake_run):
    vals = rh._counter(fake_run, "fetch", "FETCH_SIZE", "fa_fwd_kernel", STEPS, WARM)
    assert len(vals) == STEPS and set(vals.values()) == {100000.0}
    assert len(rh._counter(fake_run, "fetch", "FETCH_SIZE", "fa_fwd_kernel")) == WARM + STEPS + 5


def test_every_pass_runs_the_benchmark_command():
    progs = [prog for _, _, prog in rh.passes("B1-H32-N8192-d128-f16", "/tmp/x", 20, 5)]
    for prog in progs:
        assert prog[prog.index("--steps") + 1] == "20" and prog[prog.index("--warmup") + 1] == "5"
    for name, prof_args, _ in rh.passes("B1-H32-N8192-d128-f16", "/tmp/x", 20, 5):
        assert "--kernel-trace" in prof_args  # durations of the same dispatches in every pass


def test_summarize_arithmetic(fake_run, tmp_path):
    (rec,) = rh.summarize("B1-H32-N8192-d128-f16", fake_run, steps=STEPS, cmds=["rocprofv3 ..."], warmup=WARM)
    assert rec["kernel_ms_mean_timed"] == pytest.approx(1.0)
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_bytes"] == pytest.approx(100000.0 * 2 * 1024)
    assert rec["write_bytes"] == pytest.approx(66560.0 * 1024)
    assert rec["achieved_gb_per_s"] == pytest.approx(rec["bytes_per_launch"] / 1e-3 / 1e9)
    assert rec["mfma_flop_per_launch"] == pytest.approx(2 ** 40)
    assert rec["mfma_busy_fraction"] == pytest.approx(0.5)
    assert rec["unavoidable_bytes"] == 32 * (4 * 8192 * 128 * 2 + 4 * 8192)
    assert rec["tflops_from_trace"] == pytest.approx(4 * 32 * 8192 ** 2 * 128 / 1e-3 / 1e12)
    assert rec["kernel_sha256"] == rh.kernel_sha()
    rh.write_summary(rec, str(tmp_path / "summ"))
    j = json.load(open(tmp_path / "summ" / "traffic_fa_fwd_kernel_B1-H32-N8192-d128-f16.json"))
    assert j["bytes_per_launch"] == pytest.approx(rec["bytes_per_launch"])
    assert "dispatch_ms" not in j
    md = open(tmp_path / "summ" / "fa_fwd_kernel_B1-H32-N8192-d128-f16.md").read()
    assert "MFMA busy: **50.0 %**" in md
    assert rec["clock_ghz"] == pytest.approx(2.0)  # 2e6 GUI-active cycles per XCD in 1 ms
    assert "clock of the timed dispatches: 2.00 GHz" in md and "2097 TFLOP/s" in md
    assert "vector issue busy (incl. MFMA issue) 100.0 %" in md and "co-execution) 10.0 %" in md


def test_passes_keep_counters_within_one_pass_limits():
    for name, prof_args, prog in rh.passes("B1-H32-N8192-d128-f16", "/tmp/x", 20, 10):
        if "--pmc" in prof_args:
            counters = prof_args[prof_args.index("--pmc") + 1:]
            assert sum(c.startswith("SQ_") for c in counters) <= 8
            assert sum(c.startswith("GRBM_") for c in counters) <= 2
            assert len([c for c in counters if c in ("FETCH_SIZE", "WRITE_SIZE")]) <= 1
        assert "--no-cpu-baseline" in prog and "--no-steady-state" in prog


def test_backward_kernels_work_and_bytes():
    ks = rh.kernels("B2-H16-N8192-d128-bf16-causal", "bwd")
    assert [k[0] for k in ks] == ["fa_bwd_dq_kernel", "fa_bwd_dkdv_kernel"]
    per_product = 2.0 * 32 * 8192 ** 2 * 128 / 2
    assert ks[0][1] == pytest.approx(3 * per_product) and ks[1][1] == pytest.approx(4 * per_product)
    assert ks[0][2] == 32 * (6 * 8192 * 128 * 2 + 8 * 8192)
    assert rh.kernel_sha("bwd") != rh.kernel_sha("fwd")
    for name, prof_args, prog in rh.passes("B2-H16-N8192-d128-bf16-causal", "/tmp/x", 5, 2, "bwd"):
        assert prog[prog.index("--pass") + 1] == "bwd"


def test_block_sparse_variant():
    import workloads
    w = workloads.HEADLINE
    (k,) = rh.kernels(w.name, "fwd", blocks=(128, 0.25))
    m = workloads.make_block_mask(w, 128, 0.25)
    pairs = workloads.block_mask_pairs(m, w.N, 128, 128)
    assert 0.25 * w.N ** 2 < pairs < 0.3 * w.N ** 2  # about the density, plus the forced diagonal
    assert k[1] == pytest.approx(4.0 * w.d * w.B * w.H * pairs)
    assert rh.variant_tag(blocks=(128, 0.25)) == "_blocks128_p0.25" and rh.variant_tag(splits=2) == "_split2"
    for name, prof_args, prog in rh.passes(w.name, "/tmp/x", 5, 2, "fwd", blocks=(128, 0.25)):
        assert prog[prog.index("--block-density") + 1] == "0.25" and prog[prog.index("--block-size") + 1] == "128"
    # the backward: dq executes 3 products per allowed pair, dkdv 4
    dq, dkdv = rh.kernels(w.name, "bwd", blocks=(128, 0.25))
    assert dq[0] == "fa_bwd_dq_kernel" and dkdv[0] == "fa_bwd_dkdv_kernel"
    assert dq[1] == pytest.approx(6.0 * w.d * w.B * w.H * pairs)
    assert dkdv[1] == pytest.approx(8.0 * w.d * w.B * w.H * pairs)
    for name, prof_args, prog in rh.passes(w.name, "/tmp/x", 5, 2, "bwd", blocks=(128, 0.25)):
        assert prog[prog.index("--pass") + 1] == "bwd" and prog[prog.index("--block-density") + 1] == "0.25"


def test_clock_line():
    base = {"mfma_flop_per_launch": 1e12}
    assert "2.10 GHz" in rh.clock_line(dict(base, clock_ghz=2.1))
    assert "not given" in rh.clock_line({"mfma_flop_per_launch": 0.0, "clock_ghz": 4.0})
    assert "not given" in rh.clock_line(dict(base, clock_ghz=0.0))


def test_reference_copies_ignore_small_copy_dispatches():
    # three 256 MiB reference copies and one 4 KiB upload through the same copy kernel
    assert rh._reference_copies([131092.0, 131084.0, 131084.0, 4.0]) == [131092.0, 131084.0, 131084.0]
    assert rh._reference_copies([]) == []


def test_recorded_commands_run_from_the_repository_root():
    # an absolute interpreter and benchmark path (another machine's copy) become python3 and bench.py
    cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/p/kt -o kt -- "
           "/usr/local/bin/python3 /some/where/repo/bench.py --workload W --steps 20 --warmup 5")
    assert rh.display_command(cmd) == ("rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/p/kt "
                                       "-o kt -- python3 bench.py --workload W --steps 20 --warmup 5")
    # paths under this repository become relative to it
    import os
    inside = os.path.join(rh.ROOT, "gpurun_out", "x")
    assert rh.display_command(f"rocprofv3 -d {inside} -- python3 bench.py") == "rocprofv3 -d gpurun_out/x -- python3 bench.py"
