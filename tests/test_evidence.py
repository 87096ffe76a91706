"""Host logic of the rocprofv3 evidence harness, on synthetic rocprofv3 CSV files.

No GPU and no profiler: the files below stand in for what rocprofv3 writes, with
values chosen so every derived figure has a known answer.
"""

import csv
import json
import os

import pytest

from exact_attention_prefill_amd import evidence as ev

PRE = ev.KERNELS["prefill"]
SPLIT = ev.KERNELS["decode_split"]
MERGE = ev.KERNELS["decode_merge"]


def test_every_counter_set_fits_one_pass():
    for name, counters in ev.COUNTER_SETS.items():
        ev.check_counter_set(counters)  # raises if not


def test_oversized_sets_are_refused():
    with pytest.raises(ValueError):
        ev.check_counter_set([f"SQ_X{i}" for i in range(9)])
    with pytest.raises(ValueError):  # FETCH_SIZE takes 3 TCC slots, WRITE_SIZE 2: 5 > 4
        ev.check_counter_set(["FETCH_SIZE", "WRITE_SIZE"])
    with pytest.raises(ValueError):
        ev.check_counter_set(["GRBM_GUI_ACTIVE", "GRBM_COUNT", "GRBM_X"])


def test_commands_put_the_program_right_after_the_separator():
    for name in ev.ALL_PASSES:
        cmd = ev.pass_command(name, "/tmp/o", python="/usr/bin/python3")
        i = cmd.index("--")
        assert cmd[i + 1] == "/usr/bin/python3" and cmd[i + 2:i + 4] == ["-u", "bench.py"]
        assert cmd[0] == "timeout" and "rocprofv3" in cmd
        if name == "trace":
            assert "--kernel-trace" in cmd and "--pmc" not in cmd
        else:
            assert cmd[1:3] == ["-s", "KILL"] and "--kernel-trace" not in cmd and "--calibrate-copy" in cmd
            assert not {"-s", "--sys-trace", "-r", "--runtime-trace"} & set(cmd[cmd.index("rocprofv3"):i])


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _agent(path):
    _write(path, ["Agent_Type", "Cu_Count", "Simd_Per_Cu", "Num_Xcc", "Max_Engine_Clk_Fcompute"],
           [["CPU", 16, 0, 1, 0], ["GPU", 2, 4, 2, 2400]])


def _trace(path, seq):
    rows, t = [], 1000
    for name, dur in seq:
        rows.append(["KERNEL_DISPATCH", name, t, t + dur])
        t += dur + 10
    _write(path, ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)


def _pmc(path, seq):
    """seq: (name, duration ns, {counter: value}); one row per counter per dispatch."""
    rows, t = [], 1000
    for i, (name, dur, vals) in enumerate(seq):
        for c, v in vals.items():
            rows.append([i + 1, name, c, v, t, t + dur])
        t += dur + 10
    _write(path, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                  "End_Timestamp"], rows)


@pytest.fixture
def run_dir(tmp_path):
    out = str(tmp_path)
    _agent(os.path.join(out, "trace", "h", "run_agent_info.csv"))
    seq = []
    for _ in range(7):  # clock-settling steps: neither figure may include them
        seq += [(PRE, 5_000_000), (SPLIT, 777_777), (MERGE, 777_777)]
    for _ in range(ev.TRACE_WARMUP):  # warm-up steps: slower than the timed ones
        seq += [(PRE, 3_000_000), (SPLIT, 999_999), (MERGE, 999_999)]
    for _ in range(ev.TRACE_STEPS):  # the timed steps: prefill then decode (warm)
        seq += [(PRE, 2_000_000), (SPLIT, 999_999), (MERGE, 999_999)]
    seq += [(SPLIT, 15_000), (MERGE, 5_000)] * ev.TRACE_DECODE_ITERS  # cold decode
    seq += [(SPLIT, 17_000), (MERGE, 7_000)] * ev.TRACE_DECODE_ITERS  # the passes apart: not the figure
    seq += [(ev.KERNELS["read_floor"], 12_800)] * ev.TRACE_DECODE_ITERS  # the plain read
    seq += [(PRE, 9_000_000)] * 3  # later launches with the lse output: not the step's
    _trace(os.path.join(out, "trace", "h", "run_kernel_trace.csv"), seq)
    flop = 4.0 * 16 * 16384 * 16384 * 128
    rec = {"config": {"prefill": {"B": 1, "H": 16, "N": 16384, "d": 128, "causal": False}},
           "decode": {"bytes": 64_000_000}, "roofline": {"achieved": flop / 2.02e-3 / 1e12}}
    with open(os.path.join(out, "trace.log"), "w") as f:
        f.write("[bench] noise\n" + json.dumps(rec) + "\n")
    n_pmc = ev.PMC_WARMUP + ev.PMC_STEPS
    cal = ev.CALIBRATE_MIB * 1024

    def pmc_seq(counter, pre_val, split_val, copy_val):
        s = [("__amd_rocclr_copyBuffer", 100, {counter: 3.0})]
        for _ in range(5):  # clock-settling steps
            s += [(PRE, 1_000_000, {counter: 7e11}), (SPLIT, 1, {counter: 7e9}), (MERGE, 1, {counter: 7e9})]
        for _ in range(n_pmc):
            s += [(PRE, 1_000_000, {counter: pre_val}), (SPLIT, 1, {counter: 1e9}), (MERGE, 1, {counter: 1e9})]
        s += [(SPLIT, 1, {counter: split_val}), (MERGE, 1, {counter: 0.0})] * ev.PMC_DECODE_ITERS
        s += [(SPLIT, 1, {counter: 3e9}), (MERGE, 1, {counter: 3e9})] * ev.PMC_DECODE_ITERS  # passes apart
        s += [(PRE, 1_000_000, {counter: 1e12})]  # an lse launch: excluded
        s += [("__amd_rocclr_copyBuffer", 100, {counter: copy_val})] * 3
        return s

    _pmc(os.path.join(out, "fetch", "h", "run_counter_collection.csv"), pmc_seq("FETCH_SIZE", 1000.0, 500.0, cal / 2))
    _pmc(os.path.join(out, "write", "h", "run_counter_collection.csv"), pmc_seq("WRITE_SIZE", 300.0, 2.0, cal))
    # MFMA pass: GRBM_GUI_ACTIVE summed over 2 XCDs = 1.5e6 cycles each over a 1 ms dispatch
    # (1.5 GHz); 8 SIMDs busy 6e6 cycles in all = 50%; 1.875e5 MFMAs x 32 cycles / (8 x 1.5e6) = 50%;
    # both units busy 1.2e6 cycles = 10%.
    mf = [(PRE, 1_000_000, {"GRBM_GUI_ACTIVE": 3.0e6, "SQ_VALU_MFMA_BUSY_CYCLES": 6.0e6, "SQ_INSTS_MFMA": 1.875e5,
                            "SQ_VALU_MFMA_COEXEC_CYCLES": 1.2e6}),
          (SPLIT, 1, {"GRBM_GUI_ACTIVE": 1.0}), (MERGE, 1, {"GRBM_GUI_ACTIVE": 1.0})] * n_pmc
    mf += [(SPLIT, 1, {"GRBM_GUI_ACTIVE": 1.0}), (MERGE, 1, {"GRBM_GUI_ACTIVE": 1.0})] * (2 * ev.PMC_DECODE_ITERS)
    _pmc(os.path.join(out, "mfma", "h", "run_counter_collection.csv"), mf)
    # Wave pass: 1e6 wave-cycles, 30% issuing, 50% waiting to issue, 20% on counters or barriers.
    wv = [(PRE, 1_000_000, {"SQ_WAVE_CYCLES": 1.0e6, "SQ_ACTIVE_INST_ANY": 3.0e5, "SQ_WAIT_INST_ANY": 5.0e5,
                            "SQ_WAIT_ANY": 2.0e5}),
          (SPLIT, 1, {"SQ_WAVE_CYCLES": 1.0}), (MERGE, 1, {"SQ_WAVE_CYCLES": 1.0})] * n_pmc
    wv += [(SPLIT, 1, {"SQ_WAVE_CYCLES": 1.0}), (MERGE, 1, {"SQ_WAVE_CYCLES": 1.0})] * (2 * ev.PMC_DECODE_ITERS)
    _pmc(os.path.join(out, "wave", "h", "run_counter_collection.csv"), wv)
    return out


def test_summary_derivations(run_dir):
    d = ev.summarize(run_dir)
    flop = 4.0 * 16 * 16384 * 16384 * 128
    assert d["prefill_tflops"] == pytest.approx(flop / 2e-3 / 1e12)  # the 2 ms step launches only
    assert d["prefill_frac"] == pytest.approx(d["prefill_tflops"] / 2500)
    assert d["prefill_events_ms"] == pytest.approx(2.02)
    assert d["prefill_trace_vs_events"] == pytest.approx(2.0 / 2.02)
    assert d["decode_us_split_plus_merge"] == pytest.approx(20.0)  # cold calls only
    assert d["decode_gbs"] == pytest.approx(64e6 / 20e-6 / 1e9)
    assert d["read_floor_us"] == pytest.approx(12.8)
    assert d["read_floor_gbs"] == pytest.approx(64e6 / 12.8e-6 / 1e9)
    # FETCH factor 2 (copy read half), WRITE factor 1
    assert d["prefill_hbm_bytes"] == pytest.approx((1000.0 * 2 + 300.0) * 1024)
    assert d["decode_split_hbm_bytes"] == pytest.approx((500.0 * 2 + 2.0) * 1024)
    assert d["prefill_mfma_busy"] == pytest.approx(0.5)
    assert d["prefill_clock_ghz"] == pytest.approx(1.5)
    s = json.load(open(os.path.join(run_dir, "summary.json")))
    assert s["kernels"]["prefill"]["mfma_busy_from_insts"] == pytest.approx(0.5)
    assert s["kernels"]["prefill"]["coexec"] == pytest.approx(0.1)
    assert s["kernels"]["prefill"]["wave_issuing"] == pytest.approx(0.3)
    assert s["kernels"]["prefill"]["wave_waiting_issue"] == pytest.approx(0.5)
    assert s["kernels"]["prefill"]["wave_waiting_counters"] == pytest.approx(0.2)
    assert s["calibration"] == {"fetch": pytest.approx(2.0), "write": pytest.approx(1.0)}
    c = json.load(open(os.path.join(run_dir, "prefill_headline_counters.json")))
    assert c["kernel_sha"] == ev.source_hash(ev.PREFILL_SOURCES)
    assert c["hbm_bytes_per_launch"] == round((1000.0 * 2 + 300.0) * 1024)
    assert c["algorithmic_bytes_per_launch"] == 4 * 16 * 16384 * 128 * 2
    md = open(os.path.join(run_dir, "summary.md")).read()
    assert "python3 -u bench.py" in md and PRE in md
    assert "30% / 50% / 20%" in md


def test_stored_traffic_key_matches_what_bench_hashes():
    import bench

    assert [os.path.relpath(p, ev.ROOT) for p in bench.KERNEL_SOURCES] == ev.PREFILL_SOURCES
    assert bench.kernel_hash() == ev.source_hash(ev.PREFILL_SOURCES)


def test_committed_counters_match_the_prefill_sources():
    """profiles/prefill_headline_counters.json must have been taken on the prefill sources
    in the tree (bench.py reports its traffic only then): re-take it after any change."""
    import bench

    with open(bench.COUNTERS) as f:
        c = json.load(f)
    assert c["kernel_sha"] == bench.kernel_hash(), "re-run the evidence harness: the prefill sources changed"
    assert c["kernel"] == "void " + ev.KERNELS["prefill"] + "(attn::PrefillParams)"
    assert bench.measured_traffic() == c["hbm_bytes_per_launch"]


def test_workloads_summary_matches_a_synthetic_trace(tmp_path):
    """A trace laid out in the bench's order (the backward pass, then the head-size sweep
    and the workloads, each a run of its own launch form and grid; the three d = 128
    token splits one run told apart by duration): every workload's row gets its own
    dispatches, form and grid, and the bench's timing from the log line."""
    import math

    import workloads as W

    out = str(tmp_path)
    sweep = [W.PrefillCase(f"head size d={d}: B=1 H=16 N=16384 bf16 full", 1, 16, 16384, d, "bf16", False,
                           1 / math.sqrt(d)) for d in (32, 64, 96, 128, 256)]
    order = sweep + list(W.SMALL_F16 + W.GPT2_F16 + W.GPT2_SWEEP + W.DENSE_D128 + W.LONG)
    band = {4096: 500_000, 8192: 1_000_000, 16384: 1_800_000}
    rows, t, want = [["KERNEL_DISPATCH", "void attn::bwd_dkdv_kernel<1, 128, false>(attn::BwdParams)", 1, 0, 0]], 10, {}
    configs, by_d = {}, {}
    for i, c in enumerate(order):
        (sig, grid), wgs = ev._form_of(c, 256)
        dur = band[c.N] if c in W.DENSE_D128 else 20_000 + 1_000 * i
        for _ in range(3):
            rows.append(["KERNEL_DISPATCH", sig, grid, t, t + dur])
            t += dur + 10
        want[c.name] = (sig, wgs, dur / 1e3)
        if c.name.startswith("head size"):
            by_d[str(c.d)] = {"ms": dur / 1e6 * 1.01}
        else:
            configs[c.name] = {"ms": dur / 1e6 * 1.02}
    _write(os.path.join(out, ev.WORKLOADS_DIR, "run_kernel_trace.csv"),
           ["Kind", "Kernel_Name", "Grid_Size_X", "Start_Timestamp", "End_Timestamp"], rows)
    with open(os.path.join(out, ev.WORKLOADS_DIR + ".log"), "w") as f:
        f.write("[bench] a log line\n")
        f.write(json.dumps({"value": 1234.5, "configs": configs, "head_sizes": {"by_d": by_d}}) + "\n")
    md = open(ev.summarize_workloads(out)).read()
    assert "1234.5 TFLOP/s" in md and ev.source_hash(ev.PREFILL_SOURCES) in md
    table = {ln.split(" | ")[0][2:]: ln.split(" | ") for ln in md.splitlines()
             if ln.startswith("| ") and "`<" in ln and not ln.startswith("| workload |")}
    assert set(table) == set(want)
    for name, (sig, wgs, us) in want.items():
        cells = table[name]
        form = sig.replace("void attn::prefill_kernel", "").replace("(attn::PrefillParams)", "")
        assert cells[1] == f"`{form}`" and int(cells[2]) == wgs and int(cells[3]) == 3, name
        assert float(cells[4]) == pytest.approx(us, abs=0.01), name
        factor = 1.01 if name.startswith("head size") else 1.02
        assert float(cells[6].rstrip(" |")) == pytest.approx(us * factor, abs=0.01), name
