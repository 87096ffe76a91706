"""rocprofv3 evidence for the attention kernels on one MI355X.

    python -m exact_attention_prefill_amd.evidence --out DIR [--passes trace,fetch,write,mfma,lds,wave]
    python -m exact_attention_prefill_amd.evidence --out DIR --summarize-only
    python -m exact_attention_prefill_amd.evidence --out DIR --workloads [--summarize-only]

Runs ``bench.py`` under rocprofv3 once per pass -- a kernel trace, then one counter set
per run, because rocprofv3 collects a set in a single pass and refuses sets that exceed
a hardware block's counter slots -- and then reads the CSV files back and writes
``DIR/summary.md`` and ``DIR/prefill_headline_counters.json`` (the HBM traffic figure
``bench.py`` reports while the prefill sources hash to the same value).

What it derives, per attention kernel:

* dispatch time from the kernel trace.  The headline prefill (B=1, H=16, N=16384,
  d=128, bf16, full) is rated in TFLOP/s (4*B*H*N*N*d per launch) against the
  2.5 PFLOP/s dense bf16 peak; the ragged decode (B=8, H=12, d=64, fp16) in GB/s
  (K and V rows read, q and out) over split + merge, against 8 TB/s;
* HBM bytes per dispatch from FETCH_SIZE and WRITE_SIZE, each scaled by what the same
  counter reads for a plain device copy of known size made in the same process
  (``bench.py --calibrate-copy``);
* MFMA utilisation: SQ_VALU_MFMA_BUSY_CYCLES over (SIMDs x cycles), with the cycles
  from GRBM_GUI_ACTIVE per XCD and the clock from those cycles over the dispatch
  time, cross-checked by the instruction count (SQ_INSTS_MFMA x 32 cycles for the
  32x32x16 MFMA every one of these kernels uses).

``--workloads`` instead traces the default bench once (every prefill workload it times)
and writes ``DIR/prefill_workloads_kernel_trace.md``: per workload, its launch form, its
grid and the median dispatch time of its timed calls.

The parent process never touches the GPU: every pass is a child process, and the
program follows rocprofv3's ``--`` directly (the Python interpreter, no launcher).
A pass that fails ends the run; nothing is retried.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
MFMA_CYCLES = 32  # v_mfma_f32_32x32x16_{bf16,f16}: 8 passes of 4 cycles
CALIBRATE_MIB = 256
MIN_CLOCK_NS = 100_000  # shortest dispatch whose clock is derived

# bench.py arguments per pass: the trace pass times more launches; counter passes run a
# few (every dispatch is replayed per counter set).
TRACE_STEPS, TRACE_WARMUP, TRACE_DECODE_ITERS = 10, 2, 20
PMC_STEPS, PMC_WARMUP, PMC_DECODE_ITERS = 3, 1, 3

COUNTER_SETS = {
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
    "mfma": ["GRBM_GUI_ACTIVE", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
             "SQ_WAVES", "SQ_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES"],
    "lds": ["SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_WAIT_INST_LDS",
            "SQ_INSTS_VALU_TRANS_F32", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_SALU", "GRBM_GUI_ACTIVE"],
    "wave": ["SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_LDS",
             "SQ_ACTIVE_INST_MISC", "GRBM_GUI_ACTIVE"],
}
ALL_PASSES = ["trace"] + list(COUNTER_SETS)

# Counter slots per hardware block on this part (one pass), and the slots a derived
# counter takes.  A set beyond these makes rocprofv3 report "exceeds the capabilities"
# and stall, so sets are checked before any run.
BLOCK_SLOTS = {"SQ": 8, "TCC": 4, "TCP": 4, "TA": 2, "TD": 2, "GRBM": 2}
DERIVED_SLOTS = {"FETCH_SIZE": {"TCC": 3}, "WRITE_SIZE": {"TCC": 2}}

# Kernels of the headline workloads, by template signature.
KERNELS = {
    "prefill": "attn::prefill_kernel<1, 128, false, 8, 1, 2, 1>",
    "decode_split": "attn::decode_split_kernel<0, 64, 1>",
    "decode_merge": "attn::decode_merge_kernel<0, 64, 4>",
    "gqa_split": "attn::decode_split_mfma_kernel<1, 128>",
    "gqa_merge": "attn::decode_merge_kernel<1, 128, 4>",
    "bwd_delta": "attn::bwd_delta_kernel<1, 128>",
    "bwd_dq": "attn::bwd_dq_kernel<1, 128, false, 8>",
    "bwd_dkdv": "attn::bwd_dkdv_kernel<1, 128, false>",
    "read_floor": "attn::measure_read_kernel",
}
# Prefill sources whose hash keys the stored traffic figure (the same files bench.py hashes).
PREFILL_SOURCES = ["exact_attention_prefill_amd/csrc/prefill.hip", "exact_attention_prefill_amd/csrc/attn_device.h"]


def check_counter_set(counters):
    """Raise ValueError if a set needs more slots of a block than one pass has."""
    used = {}
    for c in counters:
        for blk, n in DERIVED_SLOTS.get(c, {c.split("_", 1)[0]: 1}).items():
            used[blk] = used.get(blk, 0) + n
    for blk, n in used.items():
        if n > BLOCK_SLOTS.get(blk, 0):
            raise ValueError(f"counter set {counters} needs {n} {blk} slots, one pass has {BLOCK_SLOTS.get(blk, 0)}")


def bench_args(trace: bool):
    if trace:
        return ["--steps", str(TRACE_STEPS), "--warmup", str(TRACE_WARMUP), "--no-cpu-baseline", "--decode-iters",
                str(TRACE_DECODE_ITERS), "--no-head-sizes", "--no-configs"]
    return ["--steps", str(PMC_STEPS), "--warmup", str(PMC_WARMUP), "--no-cpu-baseline", "--decode-iters",
            str(PMC_DECODE_ITERS), "--bwd-iters", "2", "--no-head-sizes", "--no-configs", "--calibrate-copy",
            str(CALIBRATE_MIB)]


def pass_command(name: str, out: str, python: str = sys.executable):
    """The command line of one pass (a list for subprocess; the program directly after --)."""
    d = os.path.join(out, name)
    if name == "trace":
        prof = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", d, "-o", "run"]
        limit = ["timeout", "-k", "10", "300"]
    else:
        counters = COUNTER_SETS[name]
        check_counter_set(counters)
        prof = ["rocprofv3", "--pmc", *counters, "--output-format", "csv", "-d", d, "-o", "run"]
        limit = ["timeout", "-s", "KILL", "120"]
    return limit + prof + ["--", python, "-u", "bench.py", *bench_args(name == "trace")]


def run_passes(out: str, passes):
    env = dict(os.environ, TMPDIR="/tmp")
    for name in passes:
        cmd = pass_command(name, out)
        print(f"[evidence] pass {name}: {' '.join(cmd)}", flush=True)
        with open(os.path.join(out, f"{name}.log"), "w") as log:
            r = subprocess.run(cmd, cwd=ROOT, env=env, stdout=log, stderr=subprocess.STDOUT)
        print(f"[evidence] pass {name} exit {r.returncode}", flush=True)
        if r.returncode != 0:
            return False
    return True


# ---- reading rocprofv3 CSV files ----

def _find(out: str, name: str, suffix: str):
    d = os.path.join(out, name)
    if not os.path.isdir(d):
        return None
    for root, _dirs, files in os.walk(d):
        for f in sorted(files):
            if f.endswith(suffix):
                return os.path.join(root, f)
    return None


def read_agent(path):
    """(CUs, SIMDs per CU, XCDs, peak MHz) of the first GPU agent."""
    for r in csv.DictReader(open(path)):
        if r.get("Agent_Type") == "GPU":
            return (int(r["Cu_Count"]), int(r["Simd_Per_Cu"]), int(r["Num_Xcc"]), float(r["Max_Engine_Clk_Fcompute"]))
    raise ValueError(f"no GPU agent in {path}")


def read_trace(path):
    """Kernel dispatches in order: [(name, duration ns)]."""
    rows = [r for r in csv.DictReader(open(path)) if r.get("Kind", "KERNEL_DISPATCH") == "KERNEL_DISPATCH"]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return [(r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) for r in rows]


def read_counters(path):
    """Dispatches in order: [(name, duration ns, {counter: value})], values summed over
    the rows rocprofv3 writes for one dispatch and counter."""
    by = {}
    for r in csv.DictReader(open(path)):
        key = int(r["Dispatch_Id"])
        e = by.setdefault(key, [r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), {}])
        e[2][r["Counter_Name"]] = e[2].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [tuple(by[k]) for k in sorted(by)]


def select(dispatches, signature, start=0, count=None):
    """Dispatches whose kernel name contains the signature, in order, sliced."""
    got = [d for d in dispatches if signature in d[0]]
    return got[start:] if count is None else got[start:start + count]


def calibration(dispatches, counter, true_kib):
    """true / measured KiB for the largest plain device copy (the calibration copy)."""
    vals = [d[2][counter] for d in dispatches if "copyBuffer" in d[0] and counter in d[2]]
    if not vals or max(vals) <= 0:
        return None
    return true_kib / max(vals)


def median_counter(dispatches, counter):
    vals = [d[2][counter] for d in dispatches if counter in d[2]]
    return statistics.median(vals) if vals else None


def mfma_utilisation(busy_cycles, grbm_active, n_simd, n_xcd):
    """Fraction of SIMD cycles with the matrix core busy; cycles are GRBM_GUI_ACTIVE per XCD."""
    cycles = grbm_active / n_xcd
    return busy_cycles / (n_simd * cycles)


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def bench_record(log_path):
    """The JSON line bench.py printed in a pass, or None."""
    if not os.path.exists(log_path):
        return None
    for line in open(log_path):
        if line.startswith("{"):
            return json.loads(line)
    return None


def summarize(out: str):
    """Write summary.md and prefill_headline_counters.json from the passes present."""
    tr_path = _find(out, "trace", "kernel_trace.csv")
    agent_path = _find(out, "trace", "agent_info.csv") or next(
        (p for p in (_find(out, n, "agent_info.csv") for n in COUNTER_SETS) if p), None)
    if agent_path is None:
        raise FileNotFoundError(f"no rocprofv3 output under {out}")
    cus, simd_per_cu, n_xcd, peak_mhz = read_agent(agent_path)
    n_simd = cus * simd_per_cu
    rec = bench_record(os.path.join(out, "trace.log"))
    trace = read_trace(tr_path) if tr_path else []
    pmc = {}
    for name in COUNTER_SETS:
        p = _find(out, name, "counter_collection.csv")
        if p:
            pmc[name] = read_counters(p)

    run_shape = {"trace": (TRACE_WARMUP, TRACE_STEPS, TRACE_DECODE_ITERS),
                 "pmc": (PMC_WARMUP, PMC_STEPS, PMC_DECODE_ITERS)}

    def kernel_slices(key, dispatches, kind):
        """The dispatches of one kernel that the figures describe.  The bench runs, in
        order: untimed clock-settling steps (as many as fit in its settle time), W
        warm-up steps and K timed steps (a prefill and a decode each), then I cold
        decode calls, then I cold calls of the two passes apart (attn_decode_split and
        attn_decode_merge: the same kernels), then the prefill launches that also write
        the log-sum-exp.  The settling steps are counted from the decode's dispatches;
        the prefill figures take the K timed launches and the decode figures the I cold
        one-call decodes."""
        sig = KERNELS[key]
        W_, K_, I_ = run_shape[kind]
        settle = len(select(dispatches, KERNELS["decode_split"])) - (W_ + K_) - 2 * I_
        if settle < 0:
            settle = 0
        if key == "prefill":
            return select(dispatches, sig, settle + W_, K_)
        if key in ("decode_split", "decode_merge"):
            return select(dispatches, sig, settle + W_ + K_, I_)
        return select(dispatches, sig)

    fc = calibration(pmc.get("fetch", []), "FETCH_SIZE", CALIBRATE_MIB * 1024)
    wc = calibration(pmc.get("write", []), "WRITE_SIZE", CALIBRATE_MIB * 1024)
    rows = {}
    for key in KERNELS:
        t = kernel_slices(key, trace, "trace")
        r = {"dispatches": len(t), "avg_us": statistics.mean(d[1] for d in t) / 1e3 if t else None,
             "min_us": min(d[1] for d in t) / 1e3 if t else None}
        f = median_counter(kernel_slices(key, pmc.get("fetch", []), "pmc"), "FETCH_SIZE")
        w = median_counter(kernel_slices(key, pmc.get("write", []), "pmc"), "WRITE_SIZE")
        if f is not None and w is not None and fc and wc:
            r["fetch_kib_raw"], r["write_kib_raw"] = f, w
            r["hbm_bytes"] = f * fc * 1024 + w * wc * 1024
        m = kernel_slices(key, pmc.get("mfma", []), "pmc")
        busy = median_counter(m, "SQ_VALU_MFMA_BUSY_CYCLES")
        grbm = median_counter(m, "GRBM_GUI_ACTIVE")
        insts = median_counter(m, "SQ_INSTS_MFMA")
        if busy is not None and grbm:
            r["mfma_busy"] = mfma_utilisation(busy, grbm, n_simd, n_xcd)
            r["mfma_insts"] = insts
            r["mfma_busy_from_insts"] = insts * MFMA_CYCLES / (n_simd * grbm / n_xcd) if insts is not None else None
            dur = statistics.median(d[1] for d in m)
            # GRBM_GUI_ACTIVE also counts the cycles around a dispatch, so the clock is
            # only meaningful for dispatches far longer than that margin.
            r["clock_ghz"] = (grbm / n_xcd) / dur if dur >= MIN_CLOCK_NS else None
            co = median_counter(m, "SQ_VALU_MFMA_COEXEC_CYCLES")
            r["coexec"] = co / (n_simd * grbm / n_xcd) if co is not None else None
        lds = kernel_slices(key, pmc.get("lds", []), "pmc")
        bank, active = median_counter(lds, "SQ_LDS_BANK_CONFLICT"), median_counter(lds, "SQ_LDS_IDX_ACTIVE")
        if bank is not None and active:
            r["lds_conflict_frac"] = bank / active
        # Wave time: the wave-cycles spent issuing, waiting to issue (a dependence or a
        # busy unit) and waiting on counters or barriers add up to SQ_WAVE_CYCLES.
        wv = kernel_slices(key, pmc.get("wave", []), "pmc")
        cyc = median_counter(wv, "SQ_WAVE_CYCLES")
        if cyc:
            for part, counter in (("issuing", "SQ_ACTIVE_INST_ANY"), ("waiting_issue", "SQ_WAIT_INST_ANY"),
                                  ("waiting_counters", "SQ_WAIT_ANY")):
                v = median_counter(wv, counter)
                r["wave_" + part] = v / cyc if v is not None else None
        rows[key] = r

    pre = rec["config"]["prefill"] if rec else {"B": 1, "H": 16, "N": 16384, "d": 128, "causal": False}
    flop = 4.0 * pre["B"] * pre["H"] * pre["N"] * pre["N"] * pre["d"] / (2 if pre["causal"] else 1)
    dec_bytes = rec["decode"]["bytes"] if rec else None
    p = rows["prefill"]
    pre_tf = flop / (p["avg_us"] * 1e-6) / 1e12 if p.get("avg_us") else None
    ds, dm = rows["decode_split"], rows["decode_merge"]
    dec_us = ds["avg_us"] + dm["avg_us"] if ds.get("avg_us") and dm.get("avg_us") else None
    dec_gbs = dec_bytes / (dec_us * 1e-6) / 1e9 if dec_us and dec_bytes else None
    alg_pre_bytes = 4 * pre["B"] * pre["H"] * pre["N"] * pre["d"] * 2
    sha = source_hash(PREFILL_SOURCES)
    # The same pass's bench line times the prefill with HIP events on its stream.
    ev_ms = flop / (rec["roofline"]["achieved"] * 1e12) * 1e3 if rec and rec.get("roofline") else None
    derived = {
        "prefill_events_ms": ev_ms,
        "prefill_trace_vs_events": (p["avg_us"] / 1e3) / ev_ms if ev_ms and p.get("avg_us") else None,
        "prefill_tflops": pre_tf, "prefill_frac": pre_tf / PEAK_BF16_TFLOPS if pre_tf else None,
        "prefill_mfma_busy": p.get("mfma_busy"), "prefill_clock_ghz": p.get("clock_ghz"),
        "prefill_mfma_insts": p.get("mfma_insts"), "prefill_mfma_insts_algorithmic": flop / (32 * 32 * 16 * 2),
        "prefill_hbm_bytes": p.get("hbm_bytes"), "prefill_algorithmic_bytes": alg_pre_bytes,
        "decode_us_split_plus_merge": dec_us, "decode_gbs": dec_gbs,
        "decode_frac": dec_gbs / PEAK_HBM_GBS if dec_gbs else None, "decode_algorithmic_bytes": dec_bytes,
        "decode_split_hbm_bytes": ds.get("hbm_bytes"),
        "read_floor_us": rows["read_floor"].get("avg_us"),
        "read_floor_gbs": dec_bytes / (rows["read_floor"]["avg_us"] * 1e-6) / 1e9
        if dec_bytes and rows["read_floor"].get("avg_us") else None,
    }
    with open(os.path.join(out, "summary.json"), "w") as f:
        json.dump({"agent": {"cus": cus, "simd_per_cu": simd_per_cu, "xcds": n_xcd, "peak_mhz": peak_mhz},
                   "calibration": {"fetch": fc, "write": wc}, "kernels": rows, "derived": derived,
                   "prefill_sha": sha}, f, indent=1)
    if p.get("hbm_bytes") is not None:
        with open(os.path.join(out, "prefill_headline_counters.json"), "w") as f:
            json.dump({"kernel": "void " + KERNELS["prefill"] + "(attn::PrefillParams)",
                       "workload": "prefill B=1 H=16 N=16384 d=128 bf16 non-causal", "kernel_sha": sha,
                       "kernel_sources": PREFILL_SOURCES, "fetch_size_kib_per_dispatch": p["fetch_kib_raw"],
                       "write_size_kib_per_dispatch": p["write_kib_raw"], "fetch_calibration": fc,
                       "write_calibration": wc, "calibration_copy_kib": CALIBRATE_MIB * 1024,
                       "hbm_bytes_per_launch": round(p["hbm_bytes"]), "algorithmic_bytes_per_launch": alg_pre_bytes},
                      f, indent=1)
            f.write("\n")
    with open(os.path.join(out, "summary.md"), "w") as f:
        f.write(render(out, rows, derived, (cus, simd_per_cu, n_xcd, peak_mhz), fc, wc, sha))
    return derived


def _fmt(x, spec):
    return "-" if x is None else format(x, spec)


def render(out, rows, derived, agent, fc, wc, sha):
    cus, spc, nx, mhz = agent
    rel = os.path.relpath(out, ROOT)
    lines = ["# rocprofv3 evidence: headline prefill, ragged decode, grouped decode, backward, read floor", "",
             f"Made by `python -m exact_attention_prefill_amd.evidence --out {rel}`, which ran, from the",
             f"repository root with TMPDIR=/tmp, one command per pass (`<out>` = `{rel}`):", "", "```"]
    for name in ALL_PASSES:
        if os.path.exists(os.path.join(out, f"{name}.log")):
            cmd = pass_command(name, "<out>", python="python3")
            lines.append(" ".join(cmd))
    lines += ["```", "",
              f"GPU: {cus} CUs x {spc} SIMDs in {nx} XCDs, peak clock {mhz:.0f} MHz. Prefill sources "
              f"(prefill.hip + attn_device.h) sha256[:16] `{sha}`; decode.hip "
              f"`{source_hash(['exact_attention_prefill_amd/csrc/decode.hip'])}`; bwd.hip "
              f"`{source_hash(['exact_attention_prefill_amd/csrc/bwd.hip'])}`.", "",
              f"HBM calibration (a plain {CALIBRATE_MIB} MiB device copy in the same process): FETCH_SIZE x "
              f"{_fmt(fc, '.4f')}, WRITE_SIZE x {_fmt(wc, '.4f')}.", "",
              "| kernel | dispatches | avg us | min us | HBM MB (cal.) | MFMA busy | by MFMA count | "
              "VALU+MFMA both busy | clock GHz | LDS conflict cycles | wave time: issuing / waiting to issue / "
              "waiting on counters or barriers |",
              "|---|---|---|---|---|---|---|---|---|---|---|"]
    for key, r in rows.items():
        hbm = r.get("hbm_bytes")
        lines.append(
            f"| `{KERNELS[key]}` | {r['dispatches']} | {_fmt(r['avg_us'], '.2f')} | {_fmt(r['min_us'], '.2f')} | "
            f"{_fmt(hbm / 1e6 if hbm is not None else None, '.2f')} | {_fmt(r.get('mfma_busy'), '.1%')} | "
            f"{_fmt(r.get('mfma_busy_from_insts'), '.1%')} | {_fmt(r.get('coexec'), '.1%')} | "
            f"{_fmt(r.get('clock_ghz'), '.2f')} | {_fmt(r.get('lds_conflict_frac'), '.1%')} | "
            f"{_fmt(r.get('wave_issuing'), '.0%')} / {_fmt(r.get('wave_waiting_issue'), '.0%')} / "
            f"{_fmt(r.get('wave_waiting_counters'), '.0%')} |")
    d = derived
    hb, ab = d["prefill_hbm_bytes"], d["prefill_algorithmic_bytes"]
    lines += ["",
              "Prefill rows are the step's timed launches (after the clock-settling and warm-up steps, before the",
              "launches that also write the log-sum-exp); decode rows are the cold calls (a 512 MiB read before each).", "",
              "## Derived", "",
              f"- prefill: {_fmt(d['prefill_tflops'], '.1f')} TFLOP/s = {_fmt(d['prefill_frac'], '.1%')} of "
              f"{PEAK_BF16_TFLOPS:.0f} TFLOP/s (trace average); MFMA busy {_fmt(d['prefill_mfma_busy'], '.1%')} at "
              f"{_fmt(d['prefill_clock_ghz'], '.2f')} GHz; MFMA instructions {_fmt(d['prefill_mfma_insts'], '.4g')} vs "
              f"{d['prefill_mfma_insts_algorithmic']:.4g} for the algorithmic flop",
              f"- prefill, the same pass's bench line (HIP events on the launch stream): "
              f"{_fmt(d['prefill_events_ms'], '.4f')} ms per launch; trace average / events = "
              f"{_fmt(d['prefill_trace_vs_events'], '.4f')}",
              f"- prefill HBM: {_fmt(hb / 1e6 if hb else None, '.1f')} MB per launch vs {ab / 1e6:.1f} MB algorithmic "
              f"(Q, K, V in, O out): {_fmt(hb / ab if hb else None, '.2f')}x",
              f"- decode: split + merge {_fmt(d['decode_us_split_plus_merge'], '.2f')} us (kernel time) = "
              f"{_fmt(d['decode_gbs'], '.0f')} GB/s = {_fmt(d['decode_frac'], '.1%')} of {PEAK_HBM_GBS:.0f} GB/s for "
              f"{_fmt(d['decode_algorithmic_bytes'], 'd')} algorithmic bytes; split HBM "
              f"{_fmt(d['decode_split_hbm_bytes'] / 1e6 if d['decode_split_hbm_bytes'] else None, '.2f')} MB",
              f"- read floor: {_fmt(d['read_floor_us'], '.2f')} us = {_fmt(d['read_floor_gbs'], '.0f')} GB/s for the same "
              f"bytes", "",
              "## Notes", "",
              f"- `{KERNELS['read_floor']}` is the decode's read floor: a plain cold read of the ragged decode's bytes",
              "  by as many waves as the split pass has non-empty chunks, each reading one contiguous span with",
              "  non-temporal 16-byte loads (`attn_measure_read`, measurement only), against which the split pass",
              "  and the merge's dependent launch are measured.",
              f"- The clock under the headline prefill was {_fmt(d['prefill_clock_ghz'], '.2f')} GHz on this box. The",
              "  MI355X clock under this load is power-limited and differs from box to box (1.83-1.98 GHz over the",
              "  recorded runs of the same binary), and the prefill's time follows it.", ""]
    return "\n".join(lines)


WORKLOADS_DIR = "cfgtrace"


def workloads_command(out: str, python: str = sys.executable):
    """A kernel trace of the default bench (every prefill workload it times)."""
    return ["timeout", "-k", "10", "600", "rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv",
            "-d", os.path.join(out, WORKLOADS_DIR), "-o", "run", "--", python, "-u", "bench.py", "--steps", "3",
            "--warmup", "1", "--no-cpu-baseline"]


def _form_of(case, cus: int):
    """(kernel signature, grid threads) of a workload's prefill launch, and its workgroups."""
    import exact_attention_prefill_amd as ea

    p = ea.prefill_plan(case.B, case.H, case.N, case.d, case.causal, cus)
    rows = p["rows_per_wave"] * p["waves"] // p["key_groups"]
    wgs = -(-case.N // rows) * case.H * case.B
    sig = (f"void attn::prefill_kernel<{1 if case.dtype == 'bf16' else 0}, {case.d}, "
           f"{'true' if case.causal else 'false'}, {p['waves']}, {p['rows_per_wave'] // 32}, {p['stages']}, "
           f"{p['key_groups']}>(attn::PrefillParams)")
    return (sig, wgs * 64 * p["waves"]), wgs


def summarize_workloads(out: str, cus: int = 256):
    """Each prefill workload's dispatches in a kernel trace of the default bench.

    The bench runs the head-size sweep after the step and the backward pass, then the
    workloads in its own order, so each workload's dispatches form one contiguous run of
    its (kernel, grid) there; the three d = 128 token splits share one form and grid and
    run back to back, told apart by duration.  The median is over a run's last 110
    dispatches (the timed calls and, for launch-sized calls, their graph replays)."""
    import math

    sys.path.insert(0, ROOT)
    import workloads as W

    trace = os.path.join(out, WORKLOADS_DIR, "run_kernel_trace.csv")
    with open(trace) as f:
        rows = [r for r in csv.DictReader(f) if r.get("Kind", "KERNEL_DISPATCH") == "KERNEL_DISPATCH"]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    rec = None
    log_path = os.path.join(out, WORKLOADS_DIR + ".log")
    if os.path.exists(log_path):
        with open(log_path) as f:
            for line in f:
                if line.startswith("{"):
                    rec = json.loads(line)
    runs = []
    for r in rows:
        key = (r["Kernel_Name"], int(r["Grid_Size_X"]))
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if runs and runs[-1][0] == key:
            runs[-1][1].append(dur)
        else:
            runs.append([key, [dur]])
    sweep = [W.PrefillCase(f"head size d={d}: B=1 H=16 N=16384 bf16 full", 1, 16, 16384, d, "bf16", False,
                           1 / math.sqrt(d)) for d in (32, 64, 96, 128, 256)]
    order = sweep + list(W.SMALL_F16 + W.GPT2_F16 + W.GPT2_SWEEP + W.DENSE_D128 + W.LONG)
    pos = max(i for i, r in enumerate(runs) if "bwd_dkdv" in r[0][0]) + 1
    bands = {4096: (0, 700e3), 8192: (700e3, 1.4e6), 16384: (1.4e6, 1e12)}
    table = []
    for c in order:
        key, wgs = _form_of(c, cus)
        dense = c in W.DENSE_D128
        if dense and c.N != 4096:
            j = pos - 1
        else:
            j = next((i for i in range(pos, len(runs)) if runs[i][0] == key), None)
        durs = runs[j][1] if j is not None else []
        if dense:
            lo, hi = bands[c.N]
            durs = [x for x in durs if lo <= x < hi]
        if j is not None:
            pos = j + 1
        med = statistics.median(durs[-min(len(durs), 110):]) / 1e3 if durs else None
        ev = None
        if rec:
            cfg = rec.get("configs", {}).get(c.name)
            if cfg:
                ev = cfg.get("graph_ms", cfg["ms"]) * 1e3
            elif c.name.startswith("head size"):
                ev = rec["head_sizes"]["by_d"][str(c.d)]["ms"] * 1e3
        tf = c.flop / (med * 1e-6) / 1e12 if med else None
        form = key[0].replace("void attn::prefill_kernel", "").replace("(attn::PrefillParams)", "")
        table.append((c.name, form, wgs, len(durs), med, tf, ev))
    rel = os.path.relpath(out, ROOT)
    cmd = " ".join(workloads_command("<out>", python="python3"))
    head_tf = rec.get("value") if rec else None
    lines = ["# Kernel trace: every prefill workload of the default bench", "",
             f"Made by `python -m exact_attention_prefill_amd.evidence --out {rel} --workloads`, which ran, from",
             f"the repository root with TMPDIR=/tmp (`<out>` = `{rel}`):", "", "```", cmd, "```", "",
             f"Prefill sources (prefill.hip + attn_device.h) sha256[:16] `{source_hash(PREFILL_SOURCES)}`. Each",
             "workload's row holds the `attn::prefill_kernel` dispatches of its launch form and grid, taken in the",
             "order the bench runs the workloads (each one's dispatches form one contiguous run in the trace; the",
             "three d = 128 token splits share one form and grid and run back to back, told apart by duration:",
             "below 0.7 ms, 0.7-1.4 ms, above). The form (template arguments) and the grid follow from",
             f"`attn_prefill_plan` for {cus} CUs. The median is over the run's last 110 dispatches (the timed calls",
             "and, for launch-sized calls, their graph replays); flop is 4·B·H·N²·d, halved when causal. The last",
             "column is bench.py's own timing from the same run: HIP events around one call, or per call of a",
             "replayed HIP graph of 20 calls for the launch-sized workloads (their trace medians exclude the",
             "host's launch overhead too).",
             f"The headline step ran at {_fmt(head_tf, '.1f')} TFLOP/s under the tracer on this box.", "",
             "| workload | form `<dt, d, causal, waves, blocks/wave, stages, key groups>` | workgroups | "
             "dispatches in its run | trace median us (last 110) | TFLOP/s | bench us (events; graph replays where "
             "launch-sized) |",
             "|---|---|---|---|---|---|---|"]
    for name, form, wgs, n, med, tf, ev in table:
        lines.append(f"| {name} | `{form}` | {wgs} | {n} | {_fmt(med, '.2f')} | {_fmt(tf, '.1f')} | {_fmt(ev, '.2f')} |")
    speedup = rec.get("configs", {}).get("causal_speedup") if rec else None
    if speedup:
        lines += ["", f"Causal speed-up (full time over causal time, bench.py, same run): {json.dumps(speedup)}."]
    path = os.path.join(out, "prefill_workloads_kernel_trace.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--out", required=True, help="output folder for the rocprofv3 files and the summary")
    ap.add_argument("--passes", default=",".join(ALL_PASSES))
    ap.add_argument("--summarize-only", action="store_true")
    ap.add_argument("--workloads", action="store_true", help="trace every prefill workload of the default bench")
    a = ap.parse_args(argv)
    out = os.path.abspath(a.out)
    os.makedirs(out, exist_ok=True)
    if a.workloads:
        ok = True
        if not a.summarize_only:
            cmd = workloads_command(out)
            print(f"[evidence] workloads: {' '.join(cmd)}", flush=True)
            with open(os.path.join(out, WORKLOADS_DIR + ".log"), "w") as log:
                r = subprocess.run(cmd, cwd=ROOT, env=dict(os.environ, TMPDIR="/tmp"), stdout=log,
                                   stderr=subprocess.STDOUT)
            print(f"[evidence] workloads exit {r.returncode}", flush=True)
            ok = r.returncode == 0
        if ok:
            print(summarize_workloads(out), flush=True)
        return 0 if ok else 1
    passes = [p for p in a.passes.split(",") if p]
    for p in passes:
        if p not in ALL_PASSES:
            raise SystemExit(f"unknown pass {p!r}; passes: {', '.join(ALL_PASSES)}")
        if p != "trace":
            check_counter_set(COUNTER_SETS[p])
    ok = True if a.summarize_only else run_passes(out, passes)
    d = summarize(out)
    print(json.dumps({k: v for k, v in d.items() if v is not None}), flush=True)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
