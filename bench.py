"""Benchmark of the KDA hot path on one MI355X.

A step is one kda_prefill of the single-sequence workload (B=1, H=32,
T=8192, D=128, C=64, bf16 q/k/v/o and beta, fp32 g and state), inputs
already resident in HBM. The JSON line also carries:
  * the other two prefill workloads (16 packed sequences with initial states;
    one 1,048,576-token sequence at H=16), each with its own roofline;
  * a cold-cache figure for the single-sequence workload (the device's 256 MB
    last-level cache flushed by a 512 MB write before every timed call);
  * the decode workload (512 sequences x 32 heads, D=128, 64 in-place steps);
  * the output norm and gate over the prefill output;
  * the roofline of the dominant unit, and the fp64 CPU oracle timed on the
    host cores as a reference baseline.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from gated_delta_rule_103_amd import costs, inputs, kda_decode, kda_output_gate, kda_prefill  # noqa: E402
from gated_delta_rule_103_amd.kda import kda_prefill_workspace_size  # noqa: E402

PREFILL_WORKLOAD = "single_seq_8k"
DECODE_WORKLOAD = "decode_512x32"
# arithmetic of the timed prefill path (bf16 is only the I/O type)
PREFILL_DTYPE = ("fp16 MFMA (state and U split into fp16 hi+lo) + fp32 MFMA, fp32 accumulate and state; "
                 "bf16 q/k/v/o")
EXTRA_PREFILL_WORKLOADS = ("varlen_16x", "long_1m", "long_1m_slow")
# stress companions reported beside the graded workloads, labelled as such
UNGRADED_WORKLOADS = {"long_1m_slow": "ungraded stress run: long_1m's shape with slow decay"}


# Every leg's untimed warmup lasts at least this long (and at least `warmup`
# calls): a few calls after start-up run several percent slower than the
# steady state the timed region is meant to measure. --warmup-min-s overrides
# it (profiler runs, where every call is traced, set 0).
WARMUP_MIN_S = 0.25


_warmup_min_s = WARMUP_MIN_S


def _time_region(fn, steps, warmup):
    """Run warmup untimed (at least `warmup` calls and WARMUP_MIN_S seconds),
    then time exactly `steps` back-to-back calls, synchronised on both sides:
    host wall clock for the region, and one pair of events on the current
    stream (the one the library launches on) bracketing the same calls, whose
    elapsed time / steps is the average device duration of one call. Events
    between calls would add a gap to every call."""
    t_w = time.perf_counter()
    done = 0
    while done < warmup or time.perf_counter() - t_w < _warmup_min_s:
        fn()
        done += 1
        if done % 16 == 0:
            torch.cuda.synchronize()       # the host clock then tracks the device
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, a.elapsed_time(b) / steps        # s, ms per call


def bench_prefill(steps, warmup, workload=PREFILL_WORKLOAD):
    w = inputs.WORKLOADS[workload]
    p = inputs.workload_prefill(workload, device="cuda")
    B, T, H, D, C = p.q.shape[0], p.q.shape[1], w["H"], w["D"], w["C"]
    N = p.num_seqs
    out = torch.empty(B, T, H, D, dtype=torch.bfloat16, device="cuda")
    S_out = torch.empty(N, H, D, D, dtype=torch.float32, device="cuda")
    ws_n = kda_prefill_workspace_size(N, B * T, H, D, D, C, torch.bfloat16)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")

    def step():
        kda_prefill(p.q, p.k, p.v, p.g, p.beta, p.S0, out=out, S_out=S_out, cu_seqlens=p.cu_seqlens,
                    C=C, workspace=ws)

    wall, ms = _time_region(step, steps, warmup)
    tokens = B * T
    flops = costs.prefill_flops(tokens, H, C, D)
    min_bytes = costs.prefill_min_bytes(tokens, H, D, D, N, io_bytes=2, beta_bytes=2, has_s0=p.S0 is not None)
    return dict(tokens=tokens, seqs=N, wall_s=wall, ms_per_step=wall * 1e3 / steps, kernel_ms=ms,
                flops=flops, min_bytes=min_bytes, inputs=p)


def bench_prefill_cold(reps, workload=PREFILL_WORKLOAD):
    """One kda_prefill per rep with the device's last-level cache (256 MB) flushed first
    by writing a 512 MB buffer; each call timed alone with an event pair on the launch
    stream, the flush outside it. Returns the median ms per call."""
    p = inputs.workload_prefill(workload, device="cuda")
    w = inputs.WORKLOADS[workload]
    B, T, H, D, C = p.q.shape[0], p.q.shape[1], w["H"], w["D"], w["C"]
    N = p.num_seqs
    out = torch.empty(B, T, H, D, dtype=torch.bfloat16, device="cuda")
    S_out = torch.empty(N, H, D, D, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(kda_prefill_workspace_size(N, B * T, H, D, D, C, torch.bfloat16), 1), dtype=torch.uint8,
                     device="cuda")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    times = []
    for r in range(reps + 2):
        flush.fill_(r & 0xff)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        kda_prefill(p.q, p.k, p.v, p.g, p.beta, p.S0, out=out, S_out=S_out, cu_seqlens=p.cu_seqlens, C=C,
                    workspace=ws)
        b.record()
        torch.cuda.synchronize()
        if r >= 2:
            times.append(a.elapsed_time(b))
    times.sort()
    return times[len(times) // 2]


def prefill_leg(pf, workload):
    """Rate and rooflines of one timed prefill workload (a bench_prefill result)."""
    w = inputs.WORKLOADS[workload]
    k_s = pf["kernel_ms"] * 1e-3
    tflops = pf["flops"] / k_s / 1e12
    gbps = pf["min_bytes"] / k_s / 1e9
    peak_tf, peak_bw = costs.MI355X_PEAK["bf16_TFLOPs"], costs.MI355X_PEAK["hbm_GBps"]
    leg = {"sequences": pf["seqs"], "tokens": pf["tokens"], "H": w["H"],
           "gate": f"-softplus(N(0,1){w['shift']:+g})"}
    if workload in UNGRADED_WORKLOADS:
        leg["note"] = UNGRADED_WORKLOADS[workload]
    return {**leg,
            "ms_per_call": round(pf["kernel_ms"], 4),
            "mtok_per_s": round(pf["tokens"] / k_s / 1e6, 3),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak_tf, "unit": "TFLOP/s",
                         "frac": round(tflops / peak_tf, 4),
                         "traffic": measured_traffic("kda_prefill", workload),
                         "model": "12C^3+8C^2D+6CD^2 FLOP per chunk-head"},
            "roofline_hbm": {"bound": "hbm", "achieved": round(gbps, 1), "peak": peak_bw, "unit": "GB/s",
                             "frac": round(gbps / peak_bw, 4), "bytes": pf["min_bytes"],
                             "model": "algorithmic minimum bytes per launch"}}


def bench_decode(steps, warmup):
    w = inputs.WORKLOADS[DECODE_WORKLOAD]
    x = inputs.workload_decode(DECODE_WORKLOAD, device="cuda")
    S = x.state.clone()
    out = torch.empty(w["N"], w["H"], w["D"], dtype=torch.bfloat16, device="cuda")
    nsteps = w["steps"]

    def one_pass():
        for s in range(nsteps):
            kda_decode(x.q[s], x.k[s], x.v[s], x.g[s], x.beta[s], S, out=out)

    wall, ms_pass = _time_region(one_pass, steps, warmup)
    ms_step = ms_pass / nsteps
    N, H, D = w["N"], w["H"], w["D"]
    state_bytes = costs.decode_bytes_per_head(D) * N * H
    vec_bytes = costs.decode_vector_bytes(N, H, D, D)
    return dict(ms_per_token_step=ms_step, state_bytes=state_bytes, vec_bytes=vec_bytes,
                gbps_state=state_bytes / (ms_step * 1e-3) / 1e9,
                gbps_total=(state_bytes + vec_bytes) / (ms_step * 1e-3) / 1e9,
                frac_hbm=state_bytes / (ms_step * 1e-3) / 1e9 / costs.MI355X_PEAK["hbm_GBps"])


def bench_output_gate(steps, warmup, shape):
    """kda_output_gate over a prefill output of `shape` (rows, H, Dv): bf16 o and
    gate, fp32 weight, bf16 out. Bound by HBM: o and gate read once, out written once."""
    rows, H, Dv = shape
    x = inputs.output_gate(rows, H, Dv, o_io="bf16", gate_io="bf16", o_std=0.3, seed=1001, device="cuda")
    out = torch.empty_like(x.o)

    def step():
        kda_output_gate(x.o, x.gate, x.weight, out=out)

    _, ms = _time_region(step, steps, warmup)
    nbytes = rows * H * Dv * 3 * 2 + Dv * 4
    return dict(ms=ms, bytes=nbytes, gbps=nbytes / (ms * 1e-3) / 1e9)


def cpu_baseline(p, min_seconds=10.0):
    """The fp64 oracle on the whole single-sequence workload (32 heads x 8192
    tokens), repeated until about `min_seconds` of host time has been spent."""
    import oracle
    H = p.q.shape[2]
    f64 = lambda t: t.detach().cpu().double().numpy().reshape(-1, H, t.shape[-1])
    q, k, v, g = (f64(t) for t in (p.q, p.k, p.v, p.g))
    beta = p.beta.detach().cpu().double().numpy().reshape(-1, H)
    threads = oracle.default_threads(H)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.recurrent(q, k, v, g, beta, nthreads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return dict(value=q.shape[0] * reps / dt / 1e6, unit="Mtok/s", cores=threads, kind="oracle",
                sample=f"whole {PREFILL_WORKLOAD} workload ({H} heads x {q.shape[0]} tokens, fp64 "
                       f"per-token recurrence) run {reps} times, {dt:.1f} s wall")


def measured_traffic(unit, workload):
    """HBM bytes per launch recorded under profiles/ from rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs (already scaled by the copy-probe calibration), or None when
    the kernel source has changed since the counters were taken."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) != 7 or cells[0] != "traffic" or cells[1] != unit or cells[2] != workload:
                continue
            src = os.path.join(ROOT, cells[3])
            if not os.path.exists(src):
                return None
            sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
            if not sha.startswith(cells[4]):
                return None
            return int(cells[5]) + int(cells[6])
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--warmup-min-s", type=float, default=WARMUP_MIN_S,
                    help="minimum duration of each leg's untimed warmup, in seconds")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--workload", default=PREFILL_WORKLOAD, choices=["single_seq_8k", "varlen_16x", "long_1m"],
                    help="prefill workload to time (the metric is quoted on single_seq_8k)")
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="skip the other two prefill workloads and the cold-cache leg")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="after the bench, run a plain device copy of MIB MiB three times "
                         "(the known-size reference that scales HBM counter readings)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the KDA hot path runs on a single MI355X); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    global _warmup_min_s
    _warmup_min_s = max(0.0, args.warmup_min_s)

    pf = bench_prefill(args.steps, args.warmup, args.workload)
    peak_tf = costs.MI355X_PEAK["bf16_TFLOPs"]
    peak_bw = costs.MI355X_PEAK["hbm_GBps"]
    k_s = pf["kernel_ms"] * 1e-3
    tflops = pf["flops"] / k_s / 1e12
    gbps = pf["min_bytes"] / k_s / 1e9
    value = pf["tokens"] * args.steps / pf["wall_s"] / 1e6
    extra = {}
    cold_ms = None
    if not args.no_extra_workloads and args.workload == PREFILL_WORKLOAD:
        for wl in EXTRA_PREFILL_WORKLOADS:
            # the 1M-token workload's call takes ~30 ms: fewer calls
            st = max(2, args.steps // 4) if wl.startswith("long_1m") else args.steps
            r = bench_prefill(st, min(args.warmup, 2), wl)
            del r["inputs"]
            torch.cuda.empty_cache()
            extra[wl] = prefill_leg(r, wl)
            extra[wl]["steps"] = st
        cold_ms = bench_prefill_cold(max(5, args.steps // 2))
    dec = None if args.no_decode else bench_decode(max(1, args.steps // 4), 1)
    og = bench_output_gate(args.steps, args.warmup, (pf["tokens"], w_h := inputs.WORKLOADS[args.workload]["H"],
                                                     inputs.WORKLOADS[args.workload]["D"]))
    cpu = None if (args.no_cpu_baseline or args.workload != PREFILL_WORKLOAD) else cpu_baseline(pf["inputs"])

    w = inputs.WORKLOADS[args.workload]
    line = {
        "metric": "KDA prefill Mtokens/s (H=32,D=128,C=64) + decode achieved HBM GB/s vs peak",
        "value": round(value, 3),
        "unit": "Mtok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_min_s": _warmup_min_s,
        "ms_per_step": round(pf["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": PREFILL_DTYPE,
        "data": "synthetic",
        "config": {"workload": args.workload, "sequences": pf["seqs"], "tokens": pf["tokens"],
                   "H": w["H"], "Dk": w["D"], "Dv": w["D"], "C": w["C"],
                   "io": "bf16 q/k/v/o/beta, fp32 g/state",
                   "gate": f"-softplus(N(0,1)+{w['shift']:g})"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak_tf,
                     "unit": "TFLOP/s", "frac": round(tflops / peak_tf, 4),
                     "traffic": measured_traffic("kda_prefill", args.workload),
                     "kernel": "kda_prefill call (chunk_prep_kernel + chunk_scan_kernel)",
                     "model": "12C^3+8C^2D+6CD^2 FLOP per chunk-head",
                     "kernel_ms": round(pf["kernel_ms"], 4)},
        "roofline_hbm": {"bound": "hbm", "achieved": round(gbps, 1), "peak": peak_bw, "unit": "GB/s",
                         "frac": round(gbps / peak_bw, 4),
                         "bytes": pf["min_bytes"], "model": "algorithmic minimum bytes per launch"},
    }
    if cold_ms is not None:
        line["cold_cache"] = {"workload": args.workload, "ms_per_call": round(cold_ms, 4),
                              "mtok_per_s": round(pf["tokens"] / (cold_ms * 1e-3) / 1e6, 3),
                              "note": "last-level cache (256 MB) flushed by a 512 MB write before each call; "
                                      "median of single calls"}
    if extra:
        line["prefill_workloads"] = extra
    if dec is not None:
        line["decode"] = {"workload": DECODE_WORKLOAD, "ms_per_token_step": round(dec["ms_per_token_step"], 4),
                          "roofline": {"bound": "hbm", "achieved": round(dec["gbps_state"], 1),
                                       "peak": peak_bw, "unit": "GB/s",
                                       "frac": round(dec["frac_hbm"], 4),
                                       "traffic": measured_traffic("kda_decode", DECODE_WORKLOAD),
                                       "model": "8*D^2 bytes per head-step"},
                          "gbps_incl_vectors": round(dec["gbps_total"], 1)}
    line["output_gate"] = {"shape": [pf["tokens"], w_h, w["D"]], "ms_per_call": round(og["ms"], 4),
                           "roofline": {"bound": "hbm", "achieved": round(og["gbps"], 1), "peak": peak_bw,
                                        "unit": "GB/s", "frac": round(og["gbps"] / peak_bw, 4),
                                        "traffic": measured_traffic("kda_output_gate", args.workload),
                                        "model": "read o and gate, write out (bf16), once each"}}
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)
    if args.copy_probe > 0:
        copy_probe(args.copy_probe)


def copy_probe(mib):
    """A plain elementwise copy of `mib` MiB (reads mib MiB, writes mib MiB per launch)."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


if __name__ == "__main__":
    main()
