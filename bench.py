#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet forward step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload decode] [--launch graph]

One step is one forward call of the whole step (decay, read-out, delta, rank-1
write, output, optional capture, final state) over one input set of the chosen
workload, with every input already resident in HBM. Steps cycle through enough
independent input sets ("layers", each with its own state, updated in place)
that their total size is well above the 256 MB Infinity Cache, so each call
reads its state from HBM as a decode layer does in a real model, where the
other layers' traffic evicts it between steps.

The K timed steps are enqueued as one HIP graph (launch-bound decode calls are
captured in serving loops for the same reason) or, with --launch direct, one
launch at a time, bracketed by a device synchronisation on both sides; `value`
and `ms_per_step` come from the host clock over those K steps.

The kernel's per-launch duration, from which the roofline fraction is computed,
comes from HIP events on the launch stream. A graph replay carries a fixed
entry and exit cost of several microseconds, which a short replay would spread
over its few steps, so the per-launch duration is the difference of a 2K-step
and the K-step replay divided by K (the median over several pairs): the fixed
cost cancels, and the figure does not depend on K.

Prints one JSON line. The single-layer decode line (the default) also carries
one object per other workload of the headline metric: "prefill" (512-token
prefill, tokens/s), "batched_decode", "spec_verify" and "rollback", each with
its own roofline and CPU baseline, "state_copy", the library's copy kernel
(the rollback kernel, index 0) moving exactly the decode call's state bytes,
measured the same way: a reference beside the decode figure (it reads its
index before its copy, so it is no lower bound), and "tiny", the smallest
configuration (D_k = D_v =
32, 8 tokens, 2 value heads), whose call is all launch and latency
(--no-extra leaves them out). Every CPU
baseline times the oracle on one core and on all the host's cores (threads
over the independent (sequence, value head) pairs) and names the CPU.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from linear_attention_recurrence_forward_amd.workloads import (  # noqa: E402
    WORKLOADS, make_inputs)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, published
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X FP32 vector, published (packed issue)
INFINITY_CACHE_BYTES = 256 << 20
RESIDENT_TARGET_BYTES = 1 << 30  # input sets cycled per run: >= 4x the cache
METRIC = "GDN decode µs/layer + state HBM GB/s (%peak); prefill tokens/s at n_tokens=512"
KERNEL_NAME = "gdn_recurrent"      # multi-token forward calls
DECODE_KERNEL_NAME = "gdn_decode"  # one-token forward calls
SHORT_KERNEL_NAME = "gdn_short"    # 2 to 8 tokens, and 9 to 16 on small grids
NAMES = ("q", "k", "v", "g", "beta", "state_in")
# The headline line's other workloads: (name, timed steps, warm-up steps). Each
# timed region covers tens of milliseconds of GPU work whatever --steps is
# (the 512-token prefill needs a longer warm-up to reach its loaded clock).
EXTRA = (("prefill", 500, 200), ("batched_decode", 500, 50), ("spec_verify", 2000, 200),
         ("rollback", 2000, 200), ("state_copy", 2000, 200), ("tiny", 2000, 200))
MAX_WORKER_THREADS = 16  # the host CPU share of one GPU on the GPU machines


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="decode",
                    choices=sorted(WORKLOADS) + ["rollback", "state_copy"],
                    help="forward workload, or 'rollback': accepted-prefix rollback "
                         "on the spec_verify shape, or 'state_copy': the rollback "
                         "kernel on the single-layer decode shape")
    ap.add_argument("--launch", default="graph", choices=("graph", "direct"))
    ap.add_argument("--io", default="f32", choices=("f32", "bf16"),
                    help="element type of q, k, v and output (state stays f32)")
    ap.add_argument("--normalize-k", action="store_true",
                    help="L2-normalise every key row in the kernel (gdn_forward_ex)")
    ap.add_argument("--layers", type=int, default=0,
                    help="input sets to cycle through (0: enough for 1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="CPU time budget of each oracle baseline sample (half on one "
                         "core, half on all cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", "--no-prefill", dest="no_extra", action="store_true",
                    help="leave out the other workloads' objects that the "
                         "single-layer decode line carries")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB "
                         "(reference kernel for the HBM byte counters)")
    ap.add_argument("--summarize-rocprof", metavar="DIR", default=None,
                    help="write profiles/ summaries from rocprofv3 CSV output in DIR "
                         "(kt_<workload>/, pmc_FETCH_SIZE_<workload>/, "
                         "pmc_WRITE_SIZE_<workload>/ and the bench output of each run "
                         "in <same name>.log) and exit")
    ap.add_argument("--summarize-valu-counters", metavar="DIR", default=None,
                    help="write the prefill VALU/clock counter summary under profiles/ "
                         "from the two rocprofv3 counter runs in DIR (sq1/, sq2/ and "
                         "their bench output in sq1.log) and exit")
    return ap.parse_args(argv)


def built_digest() -> str:
    """The build stamp written next to libgdn.so when it was compiled: the
    digest of the sources and flags it was built from."""
    from linear_attention_recurrence_forward_amd import build
    path = os.path.join(build.LIBDIR, "libgdn.digest")
    if not os.path.exists(path):
        return ""
    with open(path) as f:
        return f.read().strip()


def check_build() -> str:
    """Digest of the library that will be timed; exits (status 3) when its build
    stamp is missing or differs from the current sources, so that a figure is
    never reported under a build it was not measured on."""
    from linear_attention_recurrence_forward_amd import build
    stamp, current = built_digest(), build.source_digest()
    if stamp != current:
        print(f"bench.py: lib/libgdn.so was built from other sources (stamp "
              f"{stamp or 'missing'}, sources {current}); rebuild it with "
              "`python -m linear_attention_recurrence_forward_amd.build`", file=sys.stderr)
        raise SystemExit(3)
    return stamp


def traffic_from_profiles(workload: str, digest: str, kernel: str = KERNEL_NAME,
                          profiles: str | None = None):
    """HBM bytes per launch measured with rocprofv3 counters for this exact
    kernel build (None when absent or taken on another build)."""
    profiles = profiles or os.path.join(ROOT, "profiles")
    path = os.path.join(profiles, f"{kernel}_{workload}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_digest") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


def _csv(path):
    """Rows of a CSV file (or of its gzip-compressed copy path + '.gz')."""
    import csv
    import gzip
    if not os.path.exists(path) and os.path.exists(path + ".gz"):
        with gzip.open(path + ".gz", "rt") as f:
            return list(csv.DictReader(f))
    with open(path) as f:
        return list(csv.DictReader(f))


def workload_info(name: str, io: str = "f32"):
    """(forward workload, kernel name, algorithmic bytes per launch, description)
    of a bench workload name; 'rollback' is the rollback copy on the
    spec_verify shape (one state slice read and written per sequence, plus the
    index array); 'state_copy' is the same copy kernel on the single-layer
    decode shape (one token, index 0): it reads and writes exactly that call's
    state bytes and nothing else, a reference beside the decode call (it
    reads its index before the copy, so it is no lower bound; the HIP
    runtime's own device-to-device copy of those bytes is slower)."""
    if name == "rollback":
        w = WORKLOADS["spec_verify"]
        return (w, "gdn_rollback_kernel", w.state_bytes() + 4 * w.n_seqs,
                "accepted-prefix rollback after " + w.description)
    if name == "state_copy":
        w = WORKLOADS["decode"]
        return (w, "gdn_rollback_kernel", w.state_bytes() + 4 * w.n_seqs,
                "state copy (rollback kernel, index 0) on the " + w.description)
    w = WORKLOADS[name]
    if w.n_tokens == 1:
        kernel = DECODE_KERNEL_NAME
    elif w.n_tokens <= 8 or (w.n_tokens <= 16 and w.n_v_heads * w.n_seqs * w.d_v <= 16384
                             and (not w.capture or w.d_k < 128)):
        kernel = SHORT_KERNEL_NAME
    else:
        kernel = KERNEL_NAME
    if io == "bf16":
        return (w, kernel, w.algorithmic_bytes(io_bytes=2),
                w.description + ", bf16 q/k/v/output")
    return w, kernel, w.algorithmic_bytes(), w.description


def summarize_rocprof(src: str, workload: str, calib_mib: int, commands: dict,
                      out_dir: str | None = None) -> str:
    """Summaries under profiles/ from rocprofv3 CSV output (see --summarize-rocprof):
    the kernel-trace statistics of every kernel, and the HBM bytes per launch of
    the workload's kernel from FETCH_SIZE / WRITE_SIZE, each scaled by what the same
    counter reads for a plain device copy of calib_mib MiB."""
    w, kernel, alg, description = workload_info(workload)
    digests = set()
    for log in (f"kt_{workload}.log", f"pmc_FETCH_SIZE_{workload}.log",
                f"pmc_WRITE_SIZE_{workload}.log"):
        with open(os.path.join(src, log)) as f:
            for ln in f:
                if ln.startswith("{"):
                    digests.add(json.loads(ln)["kernel_digest"])
    if len(digests) != 1:
        raise SystemExit(f"{workload}: profiled runs disagree on the kernel build: {digests}")
    digest = digests.pop()
    stats = _csv(os.path.join(src, f"kt_{workload}", "run_kernel_stats.csv"))
    # Per-dispatch medians from the trace (short dispatches have long tails
    # under the profiler, which pull the average up).
    durations = {}
    trace = os.path.join(src, f"kt_{workload}", "run_kernel_trace.csv")
    if os.path.exists(trace) or os.path.exists(trace + ".gz"):
        for r in _csv(trace):
            durations.setdefault(r["Kernel_Name"], []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"# {kernel}: {description}", "",
             f"kernel digest (sha256 of sources + flags) of the profiled build: `{digest}`", "",
             "## rocprofv3 --kernel-trace --stats", "", "```", commands["kt"], "```", "",
             "| kernel | calls | average µs | median µs | p10 / p90 µs | min µs | max µs | share % |",
             "|---|---|---|---|---|---|---|---|"]
    for r in stats:
        name = r["Name"].replace("|", "/")
        if len(name) > 110:
            name = name[:107] + "..."
        d = sorted(durations.get(r["Name"], []))
        med = f"{(d[(len(d) - 1) // 2] + d[len(d) // 2]) / 2:.2f}" if d else "—"
        # nearest-rank percentiles
        pct = (f"{d[max(0, math.ceil(0.1 * len(d)) - 1)]:.2f} / "
               f"{d[max(0, math.ceil(0.9 * len(d)) - 1)]:.2f}") if d else "—"
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {med} | "
                     f"{pct} | {float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} |")
    per = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = _csv(os.path.join(src, f"pmc_{ctr}_{workload}", "run_counter_collection.csv"))
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        ours = [float(r["Counter_Value"]) for r in rows if kernel in r["Kernel_Name"]]
        ref_kib = max(copies)  # the calibration copy is the largest copy
        factor = (calib_mib * 1024.0) / ref_kib  # true KiB per counted KiB
        per[ctr] = dict(mean_kib=sum(ours) / len(ours), dispatches=len(ours),
                        copy_kib=ref_kib, factor=factor)
    fetch = per["FETCH_SIZE"]["mean_kib"] * per["FETCH_SIZE"]["factor"] * 1024
    write = per["WRITE_SIZE"]["mean_kib"] * per["WRITE_SIZE"]["factor"] * 1024
    lines += ["", "## HBM bytes per launch (rocprofv3 --pmc, one counter per run)", "",
              "```", commands["fetch"], commands["write"], "```", "",
              f"The plain copy of {calib_mib} MiB (`__amd_rocclr_copyBuffer`) reads and "
              f"writes {calib_mib} MiB; each counter is scaled by what it reads for that copy.",
              "", f"| counter | {kernel} KiB/dispatch (raw) | copy KiB (raw) | scale | "
              "bytes/launch |", "|---|---|---|---|---|"]
    for ctr, b in (("FETCH_SIZE", fetch), ("WRITE_SIZE", write)):
        d = per[ctr]
        lines.append(f"| {ctr} | {d['mean_kib']:.1f} | {d['copy_kib']:.1f} | "
                     f"{d['factor']:.4f} | {b:,.0f} |")
    lines += ["", f"Total HBM traffic per launch: {fetch + write:,.0f} B; algorithmic: "
              f"{alg:,} B (ratio {(fetch + write) / alg:.3f}).", ""]
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    md = os.path.join(out_dir, f"{kernel}_{workload}.md")
    with open(md, "w") as f:
        f.write("\n".join(lines))
    rec = dict(kernel=kernel, workload=workload, kernel_digest=digest,
               hbm_bytes_per_launch=fetch + write, fetch_bytes=fetch, write_bytes=write,
               algorithmic_bytes=alg, counters=per, calibration_copy_mib=calib_mib)
    with open(os.path.join(out_dir, f"{kernel}_{workload}_hbm_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    return md


def summarize_default_trace(src: str, command: str, out_dir: str | None = None) -> str:
    """Kernel-trace summary of the default bench command (every workload of
    the headline line in one process) from rocprofv3 CSV output in
    src/kt_default, next to the per-launch kernel times the same run's bench
    line reports (those are event timings under the profiler, which
    serialises dispatches, so they are not the unprofiled figures)."""
    stats = _csv(os.path.join(src, "kt_default", "run_kernel_stats.csv"))
    durations = {}
    for r in _csv(os.path.join(src, "kt_default", "run_kernel_trace.csv")):
        durations.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    line = None
    with open(os.path.join(src, "kt_default.log")) as f:
        for ln in f:
            if ln.startswith("{"):
                line = json.loads(ln)
    lines = ["# All kernels of the default bench line (decode, prefill, batched decode, "
             "spec verify, rollback, state copy, tiny)", "",
             f"kernel digest (sha256 of sources + flags) of the profiled build: "
             f"`{line['kernel_digest']}`", "", "```", command, "```", "",
             "| kernel | calls | average µs | median µs | min µs | share % |",
             "|---|---|---|---|---|---|"]
    for r in stats:
        name = r["Name"].replace("|", "/")
        if len(name) > 110:
            name = name[:107] + "..."
        d = sorted(durations.get(r["Name"], []))
        med = f"{(d[(len(d) - 1) // 2] + d[len(d) // 2]) / 2:.2f}" if d else "—"
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {med} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    lines += ["", "Per-launch kernel time reported by the same (profiled) run's bench line:", "",
              "| workload | kernel_us under the profiler |", "|---|---|",
              f"| decode | {line['kernel_us']:.3f} |"]
    for k in ("prefill", "batched_decode", "spec_verify", "rollback", "state_copy", "tiny"):
        if k in line:
            lines.append(f"| {k} | {line[k]['kernel_us']:.3f} |")
    lines.append("")
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    path = os.path.join(out_dir, "all_kernels_default_bench_line.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    return path


def host_cpu() -> dict:
    """The host CPU: model name, logical CPUs, the CPUs this process may run
    on, and the worker threads the all-core baseline uses (at most the CPU
    share of one GPU)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (
        os.cpu_count() or 1)
    return dict(model=model, nproc=os.cpu_count() or 1, usable=usable,
                threads=max(1, min(usable, MAX_WORKER_THREADS)))


def _timed_calls(fn, budget_s: float):
    """Call fn until budget_s has passed (at least once); (calls, seconds)."""
    calls, t0 = 0, time.perf_counter()
    while True:
        fn()
        calls += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s:
            return calls, dt


def cpu_baseline(w, budget_s: float, rollback: bool = False):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    on one thread (whole calls, or a prefix of the sequences when one call
    would exceed half the budget), then on all the host's cores (the same
    oracle loop over disjoint ranges of (sequence, value head) pairs, one range
    per thread, whole calls). Rates in the benchmark's unit: tokens/s for the
    prefill, algorithmic GB/s otherwise. rollback: the oracle's rollback copy
    on the spec_verify shape."""
    import numpy as np
    import oracle
    cpu = host_cpu()
    half = budget_s / 2
    if rollback:
        rng = np.random.default_rng(w.seed)
        cap = rng.standard_normal((w.n_seqs, w.n_tokens, w.n_v_heads, w.d_v, w.d_k),
                                  dtype=np.float32)
        state = np.zeros((w.n_seqs, w.n_v_heads, w.d_v, w.d_k), np.float32)
        acc = rng.integers(0, w.n_tokens, size=w.n_seqs).astype(np.uint32)
        per_call = w.state_bytes() + 4 * w.n_seqs
        c1, d1 = _timed_calls(lambda: oracle.rollback(cap, acc, state), half)
        cn, dn = _timed_calls(lambda: oracle.rollback_threads(cap, acc, state,
                                                              threads=cpu["threads"]), half)
        one = c1 * per_call / d1 / 1e9
        alln = cn * per_call / dn / 1e9
        unit = "GB/s"
        s1 = f"{c1} oracle rollback calls on the {w.name} shape, {d1:.1f} s, 1 thread"
        sn = (f"{cn} oracle rollback calls on the {w.name} shape, {dn:.1f} s, "
              f"{min(cpu['threads'], w.n_seqs)} threads over the sequences")
        used = min(cpu["threads"], w.n_seqs)
    else:
        x = make_inputs(w)
        bits = x["q_scale_bits"]
        args = {n: x[n] for n in NAMES}
        t0 = time.perf_counter()
        oracle.reference(**{n: a[:1] for n, a in args.items()}, q_scale_bits=bits,
                         capture=w.capture)
        per_seq = time.perf_counter() - t0
        seqs = max(1, min(w.n_seqs, int(half / max(per_seq, 1e-9))))
        part = {n: a[:seqs] for n, a in args.items()}
        c1, d1 = _timed_calls(lambda: oracle.reference(**part, q_scale_bits=bits,
                                                       capture=w.capture), half)
        pairs = w.n_seqs * w.n_v_heads
        used = min(cpu["threads"], pairs)
        cn, dn = _timed_calls(lambda: oracle.reference_threads(
            **args, q_scale_bits=bits, capture=w.capture, threads=used), half)
        if w.name == "prefill":
            unit = "tokens/s"
            one = c1 * seqs * w.n_tokens / d1
            alln = cn * w.n_seqs * w.n_tokens / dn
        else:
            unit = "GB/s"
            one = c1 * (seqs / w.n_seqs) * w.algorithmic_bytes() / d1 / 1e9
            alln = cn * w.algorithmic_bytes() / dn / 1e9
        s1 = (f"{c1} oracle call(s) over {seqs} of {w.n_seqs} sequence(s) of the {w.name} "
              f"workload, {d1:.1f} s, 1 thread")
        sn = (f"{cn} whole oracle call(s) of the {w.name} workload, {dn:.1f} s, {used} "
              f"threads over its {pairs} (sequence, value head) pairs")
    return dict(value=alln, unit=unit, cores=used, kind="oracle", sample=sn,
                single_core=dict(value=one, unit=unit, cores=1, sample=s1),
                cpu_model=cpu["model"], nproc=cpu["nproc"], usable_cpus=cpu["usable"])


VALU_PASSES = (
    "SQ_WAVES SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_VMEM_RD SQ_ACTIVE_INST_VALU "
    "SQ_ACTIVE_INST_ANY SQ_WAIT_INST_ANY SQ_BUSY_CYCLES GRBM_GUI_ACTIVE",
    "SQ_WAVES SQ_ACTIVE_INST_VALU2 SQ_INSTS_VALU_FMA_F32 SQ_INSTS_VALU_MUL_F32 "
    "SQ_INSTS_VALU_ADD_F32 SQ_INSTS_VALU_FLOPS_FP32 SQ_INSTS_LDS SQ_BUSY_CU_CYCLES "
    "GRBM_GUI_ACTIVE",
)


def summarize_valu_counters(src: str, out_dir: str | None = None) -> str:
    """The prefill VALU and clock summary from two rocprofv3 counter runs of
    the 512-token prefill (VALU_PASSES, one run each, in src/sq1 and src/sq2):
    medians over the dispatches of gdn_recurrent, the clock under load from
    GRBM_GUI_ACTIVE (summed over 8 XCDs), instructions per wave-token and the
    VALU dual-issue share (SQ_ACTIVE_INST_VALU2 counts quad-cycles that issue
    two VALU instructions)."""
    import re
    import statistics
    w = WORKLOADS["prefill"]
    med, dur, n = {}, [], 0
    for p in ("sq1", "sq2"):
        rows = {}
        for r in _csv(os.path.join(src, p, "run_counter_collection.csv")):
            if KERNEL_NAME not in r["Kernel_Name"]:
                continue
            d = rows.setdefault(r["Dispatch_Id"], {})
            d["dur"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            d[r["Counter_Name"]] = float(r["Counter_Value"])
        n = len(rows)
        for k in {k for d in rows.values() for k in d}:
            v = statistics.median(d[k] for d in rows.values())
            if k == "dur":
                dur.append(v)
            else:
                med[k] = v
    with open(os.path.join(src, "sq1.log")) as f:
        digest = re.findall(r'"kernel_digest": "([0-9a-f]+)"', f.read())[0]
    d = statistics.median(dur)
    waves, toks, simds = med["SQ_WAVES"], w.n_tokens, 1024
    cyc = med["GRBM_GUI_ACTIVE"] / 8
    qc = cyc / 4
    valu = med["SQ_INSTS_VALU"] / simds
    dual = med["SQ_ACTIVE_INST_VALU2"] / simds
    single = valu - 2 * dual
    per = lambda c: med[c] / waves / toks  # noqa: E731
    cmd = ("rocprofv3 --pmc {c} --output-format csv -d <dir>/{p} -o run -- python3 bench.py "
           "--workload prefill --steps 10 --warmup 2 --no-cpu-baseline --launch direct")
    lines = [
        f"# {KERNEL_NAME}: prefill run, VALU and clock counters (D_k=D_v={w.d_k}, "
        f"H_k={w.n_k_heads}, H_v={w.n_v_heads}, T={w.n_tokens}, S={w.n_seqs})", "",
        f"kernel digest (sha256 of sources + flags) of the profiled build: `{digest}`", "",
        "Two counter passes, each its own run (8 SQ counters and one GRBM counter per pass):",
        "", "```", cmd.format(c=VALU_PASSES[0], p="sq1"), cmd.format(c=VALU_PASSES[1], p="sq2"),
        "```", "", "Summary written by `python bench.py --summarize-valu-counters <dir>`.", "",
        f"Medians over the {n} dispatches of each run (values are summed over the chip):", "",
        "| counter | value |", "|---|---|",
        f"| dispatch duration under the profiler | {d:.1f} µs |"]
    for c in ("GRBM_GUI_ACTIVE", "SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_VALU_FMA_F32",
              "SQ_INSTS_VALU_MUL_F32", "SQ_INSTS_VALU_ADD_F32", "SQ_INSTS_VALU_FLOPS_FP32",
              "SQ_ACTIVE_INST_VALU2", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_LDS"):
        label = {"GRBM_GUI_ACTIVE": "GRBM_GUI_ACTIVE (8 XCDs)",
                 "SQ_ACTIVE_INST_VALU2": "SQ_ACTIVE_INST_VALU2 (quad-cycles issuing two VALU "
                                         "instructions)"}.get(c, c)
        lines.append(f"| {label} | {med[c]:,.0f} |")
    gflop = med["SQ_INSTS_VALU_FLOPS_FP32"] * 64 / 1e9
    lines += [
        "", f"Derived ({simds:,} SIMDs, {toks} tokens per wave):", "",
        f"- Clock under load: {med['GRBM_GUI_ACTIVE']:,.0f} / 8 XCDs = {cyc / 1e3:.1f} k cycles in "
        f"{d:.1f} µs = **{cyc / d / 1e3:.2f} GHz** (the 157.3 TFLOP/s peak assumes 2.4 GHz).",
        f"- VALU instructions per wave-token: {per('SQ_INSTS_VALU'):.1f}, of which FP32 FMA "
        f"{per('SQ_INSTS_VALU_FMA_F32'):.1f}, FP32 multiply {per('SQ_INSTS_VALU_MUL_F32'):.1f}, "
        f"FP32 add {per('SQ_INSTS_VALU_ADD_F32'):.1f}.",
        f"- Executed FP32 work: SQ_INSTS_VALU_FLOPS_FP32 x 64 lanes = {gflop:.2f} GFLOP per call "
        f"(algorithmic: {w.flops() / 1e9:.2f} GFLOP, 7 flops per cell and token).",
        f"- Issue per SIMD: {valu / 1e3:.1f} k VALU instructions in {qc / 1e3:.1f} k quad-cycles; "
        f"{dual / 1e3:.1f} k quad-cycles issue two ({2 * dual / valu * 100:.0f}% of VALU "
        f"instructions are dual-issued), {single / 1e3:.1f} k issue one, so a VALU issues in "
        f"{(dual + single) / qc * 100:.0f}% of quad-cycles; all dual-issued would need "
        f"{valu / 2 / 1e3:.1f} k.", ""]
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    path = os.path.join(out_dir, f"{KERNEL_NAME}_prefill_valu_counters.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    return path


def measure(name: str, *, steps: int, warmup: int, launch: str = "graph", io: str = "f32",
            normalize_k: bool = False, layers: int = 0, calibrate_copy_mib: int = 0,
            digest: str = ""):
    """One workload's timed run on cuda:0 (see the module doc). Returns the
    measurement as a dict (without CPU baseline)."""
    import torch
    import linear_attention_recurrence_forward_amd as gdn

    dev = torch.device("cuda:0")
    rollback = name in ("rollback", "state_copy")
    if (io == "bf16" or normalize_k) and rollback:
        raise SystemExit("bench.py: --io bf16 and --normalize-k apply to forward workloads")
    bf16 = io == "bf16"
    w, kernel_name, alg_bytes, description = workload_info(name, io)
    x = make_inputs(w)
    bits = x["q_scale_bits"]
    layers = layers or max(2, math.ceil(RESIDENT_TARGET_BYTES / max(alg_bytes, 1)))
    layers = min(layers, 4096)

    # Resident input sets: same values, distinct memory (state updated in place).
    host = {n: torch.from_numpy(x[n]) for n in NAMES}
    if bf16:
        for n in ("q", "k", "v"):
            host[n] = host[n].to(torch.bfloat16)
    sets = []
    for _ in range(layers):
        d = {n: host[n].to(dev) for n in NAMES}
        d["output"] = torch.empty(x["v"].shape, device=dev,
                                  dtype=torch.bfloat16 if bf16 else torch.float32)
        d["capture"] = (torch.empty((w.n_seqs, w.n_tokens, w.n_v_heads, w.d_v, w.d_k),
                                    device=dev) if w.capture or rollback else None)
        sets.append(d)
    params = gdn.params_for(sets[0]["q"], sets[0]["v"], bits)
    if rollback:
        # Fill every set's capture with a real forward call, then pick per
        # sequence a token to roll back to (all inside the call).
        rng = torch.Generator().manual_seed(w.seed)
        for d in sets:
            gdn.gdn_forward_capture(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                    d["state_in"], d["output"], d["state_in"],
                                    d["capture"], params)
            d["accepted"] = torch.randint(0, w.n_tokens, (w.n_seqs,), generator=rng,
                                          dtype=torch.int32).to(dev)
        torch.cuda.synchronize()

    stream = torch.cuda.Stream(dev)

    def launch_one(i):
        d = sets[i % layers]
        if rollback:
            gdn.gdn_rollback(d["capture"], d["accepted"], d["state_in"], params, stream)
        elif normalize_k:
            gdn.gdn_forward_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state_in"],
                               d["output"], d["state_in"], d["capture"], params,
                               gdn.OPT_NORMALIZE_K | (gdn.OPT_BF16_IO if bf16 else 0),
                               stream)
        elif bf16:
            gdn.gdn_forward_bf16(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state_in"],
                                 d["output"], d["state_in"], d["capture"], params, stream)
        elif w.capture:
            gdn.gdn_forward_capture(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                    d["state_in"], d["output"], d["state_in"],
                                    d["capture"], params, stream)
        else:
            gdn.gdn_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state_in"],
                            d["output"], d["state_in"], params, stream)

    torch.cuda.synchronize()

    def enqueue(n, offset):
        if launch == "graph":
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                with torch.cuda.graph(graph, stream=stream):
                    for i in range(n):
                        launch_one(offset + i)
            torch.cuda.synchronize()
            return graph.replay
        return lambda: [launch_one(offset + i) for i in range(n)]

    def events(run, ev0=None, ev1=None):
        """Seconds between HIP events recorded on the launch stream around run()
        (events created here unless given)."""
        ev0 = ev0 or torch.cuda.Event(enable_timing=True)
        ev1 = ev1 or torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            ev0.record(stream)
            run()
            ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / 1e3

    run_warm = enqueue(warmup, 0) if warmup > 0 else (lambda: None)
    run_timed = enqueue(steps, warmup)
    with torch.cuda.stream(stream):
        run_warm()
    torch.cuda.synchronize()

    # The timed region: exactly `steps` steps, synchronised on both sides.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()  # barrier: one rank only
    t0 = time.perf_counter()
    event_s = events(run_timed, ev0, ev1)
    wall = time.perf_counter() - t0

    # Per-launch kernel duration: graph replays of 2K and K steps, differenced.
    # Each pair has its own two graphs, which continue the walk through the
    # ring of input sets where the timed region left it. All graphs are
    # replayed once untimed (a graph's first launch carries set-up costs that
    # grow with its length), then again in the same order under events: the
    # walk is at least as long as the ring, so every call still finds its
    # state evicted from the caches, as in the timed region.
    if launch == "graph":
        per_rep = 3 * event_s
        reps = max(3, min(25, int(1.0 / max(per_rep, 1e-9)), 30000 // (3 * steps)))
        reps = max(reps, math.ceil(layers / (3 * steps)))
        pairs, offset = [], warmup + steps
        for _ in range(reps):
            pairs.append((enqueue(steps, offset), enqueue(2 * steps, offset + steps)))
            offset += 3 * steps
        for run_k, run_2k in pairs:
            events(run_k)
            events(run_2k)
        diffs = []
        for run_k, run_2k in pairs:
            e1 = events(run_k)
            e2 = events(run_2k)
            diffs.append((e2 - e1) / steps)
        del pairs
        kernel_s = statistics.median(diffs)
        method = (f"median over {reps} pairs of (events({2 * steps}-step replay) - "
                  f"events({steps}-step replay)) / {steps}; every replay repeated, each "
                  f"call's input set last used {reps * 3 * steps} calls before")
    else:
        kernel_s = event_s / steps
        method = f"events around the {steps} timed launches / {steps}"

    if calibrate_copy_mib:
        n = calibrate_copy_mib << 18  # floats
        a = torch.ones(n, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    ms_per_step = wall * 1e3 / steps
    if w.name == "prefill" and not rollback:
        value = w.n_seqs * w.n_tokens * steps / wall
        unit = "tokens/s"
        achieved = w.flops() / kernel_s / 1e12
        roofline = dict(bound="alu", achieved=achieved, peak=FP32_VECTOR_PEAK_TFLOPS,
                        unit="TFLOP/s", frac=achieved / FP32_VECTOR_PEAK_TFLOPS)
    else:
        value = alg_bytes * steps / wall / 1e9
        unit = "GB/s"
        achieved = alg_bytes / kernel_s / 1e9
        roofline = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBPS, unit="GB/s",
                        frac=achieved / HBM_PEAK_GBPS)
    roofline["traffic"] = (None if bf16 or normalize_k else
                           traffic_from_profiles(name, digest, kernel_name))
    roofline["kernel"] = kernel_name
    roofline["kernel_us"] = kernel_s * 1e6
    roofline["kernel_us_method"] = method
    return dict(
        name=name, w=w, bf16=bf16, rollback=rollback, value=value, unit=unit, steps=steps,
        warmup=warmup, ms_per_step=ms_per_step, event_us_per_step=event_s * 1e6 / steps,
        kernel_us=kernel_s * 1e6, roofline=roofline, description=description,
        bits=bits, layers=layers, alg_bytes=alg_bytes,
        state_gbps=w.state_bytes() / kernel_s / 1e9)


def progress(m: dict) -> None:
    """One progress line on stderr per measured workload."""
    r = m["roofline"]
    print(f"bench: {m['name']}: {m['ms_per_step'] * 1e3:.2f} us per step (host clock), "
          f"kernel {m['kernel_us']:.3f} us, {r['achieved']:.1f} {r['unit']} = "
          f"{r['frac']:.3f} of peak", file=sys.stderr, flush=True)


def extra_object(m: dict, cpu: dict | None) -> dict:
    """A non-headline workload's measurement as an object of the bench line."""
    w = m["w"]
    obj = {"metric": ("prefill tokens/s at n_tokens=512" if m["unit"] == "tokens/s" else
                      "µs per call + algorithmic HBM GB/s (%peak)"),
           "value": m["value"], "unit": m["unit"], "steps": m["steps"],
           "warmup": m["warmup"], "ms_per_step": m["ms_per_step"],
           "us_per_call": m["ms_per_step"] * 1e3, "kernel_us": m["kernel_us"],
           "workload": m["description"],
           "shape": {"d_k": w.d_k, "d_v": w.d_v, "n_k_heads": w.n_k_heads,
                     "n_v_heads": w.n_v_heads, "n_tokens": w.n_tokens,
                     "n_seqs": w.n_seqs, "q_scale_bits": m["bits"], "capture": w.capture},
           "algorithmic_bytes_per_step": m["alg_bytes"],
           "roofline": m["roofline"]}
    if m["unit"] == "GB/s":
        obj["state_gbps"] = m["state_gbps"]
    if cpu is not None:
        obj["cpu_baseline"] = cpu
    return obj


def main(argv=None):
    args = parse_args(argv)
    if args.summarize_valu_counters:
        print(summarize_valu_counters(args.summarize_valu_counters))
        return 0
    if args.summarize_rocprof:
        cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/kt_{w} -o run "
               "-- python3 bench.py --workload {w} --steps 200 --warmup 20 --no-cpu-baseline "
               "--no-extra")
        pmc = ("rocprofv3 --pmc {c} --output-format csv -d <dir>/pmc_{c}_{w} -o run -- "
               "python3 bench.py --workload {w} --steps 10 --warmup 2 --layers 4 "
               "--no-cpu-baseline --no-extra --launch direct --calibrate-copy-mib 1024")
        for wl in sorted(WORKLOADS) + ["rollback"]:
            if os.path.isdir(os.path.join(args.summarize_rocprof, f"kt_{wl}")):
                print(summarize_rocprof(args.summarize_rocprof, wl, 1024, dict(
                    kt=cmd.format(w=wl), fetch=pmc.format(c="FETCH_SIZE", w=wl),
                    write=pmc.format(c="WRITE_SIZE", w=wl))))
        if os.path.isdir(os.path.join(args.summarize_rocprof, "kt_default")):
            print(summarize_default_trace(
                args.summarize_rocprof,
                "rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/kt_default -o run "
                "-- python3 bench.py --steps 20 --warmup 5 --no-cpu-baseline"))
        return 0
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (got --gpus {args.gpus}); "
              "the op shards over sequences and value heads without any exchange, "
              "so a multi-GPU figure would be N independent copies of this one.",
              file=sys.stderr)
        return 2
    digest = check_build()

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(torch.device("cuda:0"))

    plain = args.io == "f32" and not args.normalize_k
    m = measure(args.workload, steps=args.steps, warmup=args.warmup, launch=args.launch,
                io=args.io, normalize_k=args.normalize_k, layers=args.layers,
                calibrate_copy_mib=args.calibrate_copy_mib, digest=digest)
    progress(m)
    w = m["w"]
    line = {
        "metric": METRIC,
        "value": m["value"],
        "unit": m["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if not m["bf16"] else "bf16 q/k/v/output, f32 state and arithmetic",
        "data": "synthetic",
        "config": {
            "workload": m["description"],
            "d_k": w.d_k, "d_v": w.d_v, "n_k_heads": w.n_k_heads, "n_v_heads": w.n_v_heads,
            "n_tokens": w.n_tokens, "n_seqs": w.n_seqs, "q_scale_bits": m["bits"],
            "capture": w.capture, "normalize_k": args.normalize_k,
            "launch": args.launch, "resident_sets": m["layers"],
            "algorithmic_bytes_per_step": m["alg_bytes"],
            "flops_per_step": 0 if m["rollback"] or m["name"] == "state_copy" else w.flops(),
        },
        "us_per_layer": m["ms_per_step"] * 1e3,
        "kernel_us": m["kernel_us"],
        "event_us_per_step": m["event_us_per_step"],
        "state_gbps": m["state_gbps"],
        "roofline": m["roofline"],
        "kernel_digest": digest,
    }
    extras = []
    if args.workload == "decode" and plain and not args.no_extra:
        # The metric's other workloads, measured the same way in the same process.
        for name, steps, warmup in EXTRA:
            extras.append(measure(name, steps=steps, warmup=warmup, launch=args.launch,
                                  digest=digest))
            progress(extras[-1])
            torch.cuda.empty_cache()
    # CPU baselines after all GPU work (they share nothing with it).
    if not args.no_cpu_baseline and plain:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, rollback=m["rollback"])
    for e in extras:
        # The state copy is a reference point, not a workload of the metric.
        cpu = (None if args.no_cpu_baseline or e["name"] == "state_copy" else
               cpu_baseline(e["w"], args.cpu_seconds, rollback=e["rollback"]))
        line[e["name"]] = extra_object(e, cpu)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
