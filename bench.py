"""Benchmark of the attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the whole hot path over one batch of synthetic input:
  * prefill at the headline shape: B=1, H=16, N=16384, d=128, bf16, non-causal,
    scale 1/sqrt(128) (the dense d=128 comparison on page 1 at 16K tokens);
  * decode over the ragged batch: B=8, H=12, d=64, fp16, cache 4096 rows, lengths
    uniform in [1, 4096] from seed 0 (page 3, "What can it do": a different current
    length per sequence), split-K with the automatic chunk, then the merge.
Inputs are made once from seed 0 and are resident in HBM before timing starts.
100 ms of untimed steps settle the clock (input generation leaves the GPU idle), then W
untimed steps, then K timed steps between two device synchronisations.

Prints ONE JSON line.  `value` is prefill TFLOP/s over the whole timed region
(algorithmic flop 4*B*H*N*N*d per step / wall time per step, decode included in the
time).  `roofline` covers the prefill kernel, timed with HIP events on the stream it
runs on.  `decode` reports the decode path's HBM rate, timed with events after a
512 MiB read that evicts the L2 and the Infinity Cache before every call.
It also times the two passes apart (`split_us_cold`, `merge_us`: events at the
boundaries of attn_decode_split and attn_decode_merge) and, as the floor the split pass
is measured against, a plain cold read of the same bytes (`read_floor`).
`decode_gqa` does the same for grouped K/V heads (B=8, 32 query heads over 8 K/V
heads of 128, bf16, cache 4096 rows), whose bytes count the cache once per K/V head;
it runs after the timed steps and is not part of them.
`backward` times the backward pass (dq, dk, dv from out, lse and a seeded dout) at
the prefill's shape, also outside the steps and once the clock settles (as the
prefill with the log-sum-exp output, `prefill_lse`); its flop count is 2.5 times the
forward's (the five products of the chain rule, each of the forward's size).
`head_sizes` times the prefill at d = 32, 64, 96, 128 and 256 with the headline's
B, H and N (bf16, non-causal), outside the steps.
`configs` times every other workload shape alone, outside the steps (events around
each call; the calls small enough to be launch-bound also as one HIP graph of 20
calls replayed, `graph_ms`, which leaves the host's launch overhead out): the small
prefill (B=1, H=1, N=128, d=64, fp16), the GPT-2-like prompt (B=1, H=12, N=2048, d=64,
fp16, full and causal) and its sweep (B in {1, 4} x N in {128, 512, 1024, 4096}, both
masks; `causal_speedup` is full time over causal time per shape), the dense d=128
token splits (B*N = 16384 at H=16), the long
sequences (B=1, H=24, d=128, bf16: N=32768 full, N=16384 causal) and the batch-1
decode over a full 4096-row cache, cold like the step's decode.
`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the same prefill; in
the same host leg the oracle checks this run's outputs on sampled rows (`parity`).
With --no-cpu-baseline the oracle is not imported at all and both are null.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
COUNTERS = os.path.join(ROOT, "profiles", "prefill_headline_counters.json")
KERNEL_SOURCES = [
    os.path.join(ROOT, "exact_attention_prefill_amd", "csrc", f)
    for f in ("prefill.hip", "attn_device.h")
]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per prefill launch from the committed counter runs, if they were taken
    on the current kernel source; else None."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_sha") != kernel_hash():
        return None
    return c.get("hbm_bytes_per_launch")


def cpu_baseline(q, k, v, scale, budget_s):
    """Time the fp64 oracle on whole heads of the headline prefill until budget_s passes."""
    import numpy as np
    import torch

    import oracle

    try:
        from threadpoolctl import threadpool_info

        cores = max((i.get("num_threads") or 1) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:  # threadpoolctl missing: report the host count
        cores = os.cpu_count()
    N, d = q.shape[2], q.shape[3]
    rows_per_block = 2048
    done_rows, t_total = 0, 0.0
    h = 0
    while t_total < budget_s and h < q.shape[1]:
        qh, kh, vh = (t[0, h].to(torch.float64).numpy()[None, None] for t in (q, k, v))
        for r0 in range(0, N, rows_per_block):
            rows = np.arange(r0, min(N, r0 + rows_per_block))
            t0 = time.perf_counter()
            oracle.prefill_rows(qh, kh, vh, False, scale, 0, 0, rows)
            t_total += time.perf_counter() - t0
            done_rows += len(rows)
            if t_total >= budget_s:
                break
        h += 1
    flop = 4.0 * done_rows * N * d
    return {
        "value": flop / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{done_rows} query rows (of head 0 onward) of the B=1 H=16 N=16384 d=128 bf16 non-causal "
        f"prefill, fp64 NumPy, {t_total:.1f} s",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-iters", type=int, default=100)
    ap.add_argument("--bwd-iters", type=int, default=10)
    ap.add_argument("--no-head-sizes", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip timing every workload shape")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument(
        "--calibrate-copy",
        type=int,
        default=0,
        metavar="MIB",
        help="after measuring, copy a MIB-sized buffer three times (a plain copy kernel of known "
        "size that calibrates the HBM byte counters in a profiled run)",
    )
    args = ap.parse_args()
    if args.gpus != 1:
        print(
            f"bench.py measures one GPU only: the attention forward here is a single-GPU kernel library "
            f"(--gpus {args.gpus} is not supported; run with --gpus 1)",
            file=sys.stderr,
        )
        sys.exit(2)

    import numpy as np
    import torch

    import exact_attention_prefill_amd as ea
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    cus = props.multi_processor_count

    P = W.HEADLINE
    log(f"device {props.name} ({getattr(props, 'gcnArchName', '?')}), {cus} CUs; making inputs")
    qc, kc, vc = W.prefill_inputs(P.B, P.H, P.N, P.d, P.dtype, seed=0)
    q, k, v = (t.to(dev) for t in (qc, kc, vc))
    out = torch.empty_like(q)

    D = W.DECODE[1]
    dq, dk, dv, dl = W.decode_inputs(D.B, D.H, D.max_len, D.d, D.dtype, seed=0)
    dq_, dk_, dv_, dl_ = (t.to(dev) for t in (dq, dk, dv, dl))
    dout = torch.empty_like(dq_)
    chunk, n_split = ea.decode_choose_split(D.B, D.H, D.max_len, D.d, cus)
    ws = torch.empty(ea.decode_workspace_bytes(D.B, D.H, n_split, D.d), dtype=torch.uint8, device=dev)
    dec_bytes = W.decode_bytes(D.H, D.d, dl.tolist())

    def step(ev=None):
        if ev:
            ev[0].record()
        ea.prefill(q, k, v, causal=P.causal, scale=P.scale, out=out)
        if ev:
            ev[1].record()
        ea.decode(dq_, dk_, dv_, dl_, scale=D.scale, out=dout, chunk=chunk, workspace=ws)
        if ev:
            ev[2].record()

    # Making the inputs on the host leaves the GPU idle for seconds, and its clock drops;
    # 100 ms of untimed steps bring it back to the steady state before the W warm-up
    # steps and the K timed ones.
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) < 0.1:
        step()
        torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dec_ms_warm = [e[1].elapsed_time(e[2]) for e in evs]
    ms_per_step = wall * 1e3 / args.steps
    pre_mean = float(np.mean(pre_ms))
    pre_tflops = P.flop / (pre_mean * 1e-3) / 1e12
    value = P.flop / (ms_per_step * 1e-3) / 1e12
    log(f"prefill {pre_mean:.3f} ms/launch = {pre_tflops:.1f} TFLOP/s; step {ms_per_step:.3f} ms")

    # Decode, cold: evict L2 and the 256 MB Infinity Cache by reading 512 MiB first.
    # A read leaves clean lines behind; a write-based flush would leave ~256 MB of
    # dirty lines whose write-back then competes with the decode's reads.
    flush = torch.ones(128 << 20, dtype=torch.int32, device=dev)
    flush_sink = torch.empty((), dtype=torch.int64, device=dev)

    def cold_us_of(call, iters):
        cold = []
        for _ in range(iters):
            torch.sum(flush, dim=0, out=flush_sink)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            b.record()
            cold.append((a, b))
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in cold])) * 1e3

    cold_us = cold_us_of(lambda: ea.decode(dq_, dk_, dv_, dl_, scale=D.scale, out=dout, chunk=chunk, workspace=ws),
                         args.decode_iters)
    warm_us = float(np.mean(dec_ms_warm)) * 1e3
    dec_gbs = dec_bytes / (cold_us * 1e-6) / 1e9
    log(f"decode cold {cold_us:.2f} us = {dec_gbs:.0f} GB/s; warm {warm_us:.2f} us")

    # The two passes apart (attn_decode_split, then attn_decode_merge on the partials it
    # left), cold as above; and the floor the split pass is measured against: a plain cold
    # read of the same bytes by as many waves as the split has non-empty chunks, each
    # reading one contiguous span (attn_measure_read).
    def passes_cold(iters):
        spans = []
        for _ in range(iters):
            torch.sum(flush, dim=0, out=flush_sink)
            a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            a.record()
            ea.decode_split(dq_, dk_, dv_, dl_, D.scale, chunk, ws)
            b.record()
            ea.decode_merge(ws, dout, D.max_len, chunk)
            c.record()
            spans.append((a, b, c))
        torch.cuda.synchronize()
        return (float(np.mean([a.elapsed_time(b) for a, b, _ in spans])) * 1e3,
                float(np.mean([b.elapsed_time(c) for _, b, c in spans])) * 1e3)

    split_us, merge_us = passes_cold(args.decode_iters)
    live_waves = D.H * sum(-(-int(L) // chunk) for L in dl.tolist())
    read_buf = torch.empty((dec_bytes + 15) // 16 * 16, dtype=torch.uint8, device=dev)
    read_sink = torch.zeros(live_waves * 64, dtype=torch.int32, device=dev)
    read_us = cold_us_of(lambda: ea.measure_read(read_buf, live_waves, read_sink), args.decode_iters)
    del read_buf
    log(f"decode passes cold: split {split_us:.2f} us, merge {merge_us:.2f} us (events at the pass boundaries); "
        f"plain read of the same bytes by {live_waves} waves {read_us:.2f} us = "
        f"{dec_bytes / (read_us * 1e-6) / 1e9:.0f} GB/s")

    # Grouped K/V heads (a wider row than the step: the K/V cache is read once per
    # group of query heads), timed the same way outside the step.
    GQ = W.DECODE_GQA[0]
    gkv = W.DECODE_GQA_HKV[GQ.name]
    gq, gk, gv, gl = W.decode_inputs_gqa(GQ.B, GQ.H, gkv, GQ.max_len, GQ.d, GQ.dtype, seed=0)
    gq_, gk_, gv_, gl_ = (t.to(dev) for t in (gq, gk, gv, gl))
    gout = torch.empty_like(gq_)
    gchunk, gns = ea.decode_gqa_choose_split(GQ.B, GQ.H, gkv, GQ.max_len, GQ.d, cus)
    gws = torch.empty(ea.decode_workspace_bytes(GQ.B, GQ.H, gns, GQ.d), dtype=torch.uint8, device=dev)
    gcall = lambda: ea.decode(gq_, gk_, gv_, gl_, scale=GQ.scale, out=gout, chunk=gchunk, workspace=gws)  # noqa: E731
    for _ in range(3):
        gcall()
    gqa_us = cold_us_of(gcall, args.decode_iters)
    gqa_bytes = W.decode_bytes(GQ.H, GQ.d, gl.tolist(), Hkv=gkv)
    gqa_gbs = gqa_bytes / (gqa_us * 1e-6) / 1e9
    log(f"decode (grouped heads {GQ.H}/{gkv}) cold {gqa_us:.2f} us = {gqa_gbs:.0f} GB/s")

    def settled_ms(call, n=10, warm_ms=80.0):
        """Median event time of n calls, after calling for warm_ms of wall time first:
        making each shape's inputs on the host leaves the GPU idle long enough for its
        clock to drop, and a couple of warm-up calls do not bring it back."""
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < warm_ms:
            call()
            torch.cuda.synchronize()
        evs_ = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs_:
            a.record()
            call()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs_]))

    # The prefill with its row log-sum-exp output (the forward the backward pass needs),
    # after its clock settles: the cold decode calls before it leave the GPU mostly idle.
    lse_buf = torch.empty(P.B, P.H, P.N, dtype=torch.float32, device=dev)
    lse_ms = settled_ms(lambda: ea.prefill(q, k, v, causal=P.causal, scale=P.scale, out=out, lse=lse_buf))
    log(f"prefill with lse {lse_ms:.3f} ms = {P.flop / (lse_ms * 1e-3) / 1e12:.1f} TFLOP/s")

    # Backward pass at the prefill's shape (out and lse from the forward with the
    # log-sum-exp output, a seeded dout), timed with events outside the step once its
    # clock settles (median of the calls).
    bdo = W.prefill_inputs(P.B, P.H, P.N, P.d, P.dtype, seed=1)[0].to(dev)
    bout, blse = ea.prefill(q, k, v, causal=P.causal, scale=P.scale, lse=True)
    bws = torch.empty(ea.backward_workspace_bytes(P.B, P.H, P.N) // 4, dtype=torch.float32, device=dev)
    bgrads = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]

    def bcall():
        ea.backward(q, k, v, bout, bdo, blse, causal=P.causal, scale=P.scale, dq=bgrads[0], dk=bgrads[1],
                    dv=bgrads[2], workspace=bws)

    bwd_ms = settled_ms(bcall, n=args.bwd_iters)
    bwd_flop = 2.5 * P.flop  # five products of the forward's size (QK^T, dO V^T, dV, dQ, dK)
    bwd_tflops = bwd_flop / (bwd_ms * 1e-3) / 1e12
    log(f"backward {bwd_ms:.3f} ms = {bwd_tflops:.1f} TFLOP/s")

    def graph_ms(call, reps=20, n=5, warm_ms=80.0):
        """Per-call GPU time of `reps` calls captured in one HIP graph, median of n
        replays after the clock settles: the host's launch overhead is left out, as a
        serving loop replaying a captured graph sees it.  The calls capture kernel
        launches only (no allocation, no memset)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # capture wants the calls warmed up off the default stream
            call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                call()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < warm_ms:
            g.replay()
            torch.cuda.synchronize()
        evs_ = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs_:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in evs_])) / reps
        del g
        return ms

    # Prefill at every head size the library builds, at the headline's B, H and N
    # (bf16, non-causal; flop 4*B*H*N*N*d), timed with events outside the step.
    head_sizes = {}
    if not args.no_head_sizes:
        for hd in (32, 64, 96, 128, 256):
            hq, hk, hv = (t.to(dev) for t in W.prefill_inputs(P.B, P.H, P.N, hd, "bf16", seed=0))
            hout = torch.empty_like(hq)
            hms = settled_ms(lambda: ea.prefill(hq, hk, hv, scale=1 / math.sqrt(hd), out=hout))
            htf = 4.0 * P.B * P.H * P.N * P.N * hd / (hms * 1e-3) / 1e12
            head_sizes[str(hd)] = {"ms": round(hms, 4), "tflops": round(htf, 1), "frac": round(htf / PEAK_BF16_TFLOPS, 4)}
            del hq, hk, hv, hout
        log("head sizes: " + ", ".join(f"d={k} {v['tflops']} TF" for k, v in head_sizes.items()))

    # Every prefill workload shape (small, GPT-2-like at 2048 tokens, the dense d=128
    # token splits, the long sequences) and the batch-1 decode, each timed alone with
    # events: median of 10 launches after the clock has settled; decode cold as above.
    configs = {}
    if not args.no_configs:
        for case in W.SMALL_F16 + W.GPT2_F16 + W.GPT2_SWEEP + W.DENSE_D128 + W.LONG:
            cq, ck, cv = (t.to(dev) for t in W.prefill_inputs(case.B, case.H, case.N, case.d, case.dtype, seed=0))
            cout = torch.empty_like(cq)
            ccall = lambda: ea.prefill(cq, ck, cv, causal=case.causal, scale=case.scale, out=cout)  # noqa: E731
            cms = settled_ms(ccall)
            ctf = case.flop / (cms * 1e-3) / 1e12
            configs[case.name] = {"ms": round(cms, 4), "tflops": round(ctf, 1), "frac": round(ctf / PEAK_BF16_TFLOPS, 4)}
            if case.flop < 1e11:  # launch-latency-sized calls: also their GPU time alone
                gms = graph_ms(ccall)
                gtf = case.flop / (gms * 1e-3) / 1e12
                configs[case.name].update({"graph_ms": round(gms, 4), "graph_tflops": round(gtf, 1)})
            del cq, ck, cv, cout
        # Causal tile skipping (page 3, "Kernel design" and "Performance": about 1.8-1.9x
        # at N = 4096 on its GPU): full time over causal time per GPT-2-like shape, from
        # the graph replays where the calls are launch-sized.
        speedup = {}
        for case in W.GPT2_F16 + W.GPT2_SWEEP:
            if not case.causal:
                continue
            full = configs[case.name.replace("_causal", "_full")]
            caus = configs[case.name]
            key = "graph_ms" if "graph_ms" in full and "graph_ms" in caus else "ms"
            speedup[case.name.replace("_causal", "")] = round(full[key] / caus[key], 3)
        configs["causal_speedup"] = speedup
        D1 = W.DECODE[0]
        eq, ek, ev_, el = (t.to(dev) for t in W.decode_inputs(D1.B, D1.H, D1.max_len, D1.d, D1.dtype, seed=0))
        eout = torch.empty_like(eq)
        echunk, ens = ea.decode_choose_split(D1.B, D1.H, D1.max_len, D1.d, cus)
        ews = torch.empty(ea.decode_workspace_bytes(D1.B, D1.H, ens, D1.d), dtype=torch.uint8, device=dev)
        ecall = lambda: ea.decode(eq, ek, ev_, el, scale=D1.scale, out=eout, chunk=echunk, workspace=ews)  # noqa: E731
        for _ in range(3):
            ecall()
        eus = cold_us_of(ecall, args.decode_iters)
        ebytes = W.decode_bytes(D1.H, D1.d, el.cpu().tolist())
        egbs = ebytes / (eus * 1e-6) / 1e9
        configs[D1.name] = {"us_cold": round(eus, 3), "gbs": round(egbs, 1), "frac": round(egbs / PEAK_HBM_GBS, 4),
                            "bytes": ebytes, "chunk": echunk, "n_split": ens}
        del eq, ek, ev_, eout, ews
        log("configs: " + ", ".join(f"{k} {v.get('tflops', v.get('gbs'))}" for k, v in configs.items()
                                    if k != "causal_speedup"))
        log("causal speed-up (full / causal time): " + json.dumps(configs["causal_speedup"]))

    # The host leg: the fp64 CPU oracle, run only with the CPU baseline (it is skipped
    # with --no-cpu-baseline, as in every profiled run).  It checks this run's outputs
    # on sampled rows and then times the oracle itself.
    parity = None
    if not args.no_cpu_baseline:
        import oracle

        rows = W.prefill_rows_sample(P.N, 16, 0)
        perr = 0.0
        for h in (0, P.H - 1):
            f = lambda t: t[0, h].to(torch.float64).numpy()[None, None]  # noqa: E731
            ref = oracle.prefill_rows(f(qc), f(kc), f(vc), P.causal, P.scale, 0, 0, rows)
            got = out[0, h, rows].to(torch.float64).cpu().numpy()
            perr = max(perr, float(np.max(np.abs(got - ref))))
        dref = oracle.decode(dq.double().numpy(), dk.double().numpy(), dv.double().numpy(), dl.numpy(), D.scale)
        derr = float(np.max(np.abs(dout.double().cpu().numpy() - dref)))
        gref = oracle.decode(gq.double().numpy(), gk.double().numpy(), gv.double().numpy(), gl.numpy(), GQ.scale)
        gerr = float(np.max(np.abs(gout.double().cpu().numpy() - gref)))
        bdq_rows = oracle.backward_dq_rows(qc[:, :1].double().numpy(), kc[:, :1].double().numpy(),
                                           vc[:, :1].double().numpy(), bdo[:, :1].double().cpu().numpy(),
                                           P.causal, P.scale, 0, 0, rows)
        berr = float(np.max(np.abs(bgrads[0][0, 0, rows].double().cpu().numpy() - bdq_rows)))
        log(f"parity: prefill sampled max err {perr:.2e}, decode max err {derr:.2e}, grouped decode {gerr:.2e}, "
            f"backward dq sampled {berr:.2e}")
        parity = {"prefill_sampled_max_err": perr, "decode_max_err": derr, "decode_gqa_max_err": gerr,
                  "backward_dq_sampled_max_err": berr}

    if args.calibrate_copy:
        src = torch.empty(args.calibrate_copy << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        log(f"oracle CPU baseline (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(qc, kc, vc, P.scale, args.cpu_seconds)

    traffic = measured_traffic()
    rec = {
        "metric": "prefill TFLOP/s & % MFMA peak (d=128, N=16K); decode HBM GB/s & % peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "prefill B=1 H=16 N=16384 d=128 bf16 non-causal + decode B=8 H=12 d=64 fp16 ragged cache 4096",
            "prefill": {"B": P.B, "H": P.H, "N": P.N, "d": P.d, "dtype": P.dtype, "causal": P.causal},
            "decode": {"B": D.B, "H": D.H, "max_len": D.max_len, "d": D.d, "dtype": D.dtype,
                       "seq_lens": dl.tolist(), "chunk": chunk, "n_split": n_split},
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(pre_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
        "decode": {
            "bound": "hbm",
            "achieved": round(dec_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
            "us_cold": round(cold_us, 3),
            "us_warm": round(warm_us, 3),
            "bytes": dec_bytes,
            "split_us_cold": round(split_us, 3),
            "merge_us": round(merge_us, 3),
            "read_floor": {"us_cold": round(read_us, 3), "waves": live_waves,
                           "gbs": round(dec_bytes / (read_us * 1e-6) / 1e9, 1),
                           "what": "attn_measure_read of the same bytes, one contiguous span per wave, as many "
                                   "waves as the split pass has non-empty chunks"},
        },
        "decode_gqa": {
            "bound": "hbm",
            "achieved": round(gqa_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gqa_gbs / PEAK_HBM_GBS, 4),
            "us_cold": round(gqa_us, 3),
            "bytes": gqa_bytes,
            "config": {"B": GQ.B, "Hq": GQ.H, "Hkv": gkv, "max_len": GQ.max_len, "d": GQ.d, "dtype": GQ.dtype,
                       "seq_lens": gl.tolist(), "chunk": gchunk, "n_split": gns},
        },
        "prefill_lse": {"ms": round(lse_ms, 4), "tflops": round(P.flop / (lse_ms * 1e-3) / 1e12, 1)},
        "backward": {
            "bound": "mfma",
            "achieved": round(bwd_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 4),
            "ms": round(bwd_ms, 4),
            "flop": bwd_flop,
            "config": {"B": P.B, "H": P.H, "N": P.N, "d": P.d, "dtype": P.dtype, "causal": P.causal},
        },
        "head_sizes": {"config": f"prefill B={P.B} H={P.H} N={P.N} bf16 non-causal", "by_d": head_sizes},
        "configs": configs,
        "parity": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
