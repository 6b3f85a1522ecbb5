"""rocprofv3 profiles of bench.py, one workload at a time, summarised as text.

    python3 profile_bench.py --out <dir> [--raw <dir>] [--workload 4 --workload 2 ...]

For each workload (default: all of 1 - 6) it runs, each under its own time
limit and from /tmp (TMPDIR=/tmp):

1. ``rocprofv3 --kernel-trace --stats -- python3 bench.py --workload N
   --no-cpu-baseline``: the bench exactly as timed (fused, unfused sequence,
   plain GEMM and, for norm layers, the other gain placement, round-robin, a
   cache flush before every step).  The trace is cut into steps at the flushes
   (``FillFunctor<float>`` dispatches); the last ``steps x variants`` steps
   are the timed ones, and the summary gives each variant's kernel time per
   step next to the bench's own event timings of the same run.
2. Five counter passes over ``bench.py --workload N --no-unfused
   --copy-calibration`` (the headline kernel alone): FETCH_SIZE; WRITE_SIZE;
   GRBM_GUI_ACTIVE with the MFMA and LDS counters; GRBM_GUI_ACTIVE with the
   VALU / wait counters; the instruction cache.  FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are
   scaled by 256 MiB / (the same counter for a plain 256 MiB device copy in
   the same process).  They count L2-to-fabric traffic: L2 misses, which the
   Infinity Cache or HBM serve.

Writes ``<dir>/summaries/<key>_kernel_trace.txt``, ``<key>_traffic.json``
(``bytes_per_launch``) and ``<key>_counters.json`` (``fused.clock_ghz``,
``fused.mfma_busy_pct``), each with the kernel sources' hash, which bench.py
reads from ``profiles/`` when the hash matches its sources.
"""
from __future__ import annotations

import argparse
import collections
import glob
import json
import os
import sqlite3
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (the workload names, source hash and copy size)

NUM_XCD = 8
NUM_SIMD = 256 * 4
PASSES = {
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
    "sq_mfma_lds": ["GRBM_GUI_ACTIVE", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES",
                    "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_LDS", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS",
                    "SQ_LDS_BANK_CONFLICT"],
    "sq_valu_wait": ["GRBM_GUI_ACTIVE", "SQ_WAVES", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_VMEM",
                     "SQ_ACTIVE_INST_ANY", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY"],
    "sqc_icache": ["GRBM_GUI_ACTIVE", "SQ_IFETCH", "SQC_ICACHE_REQ", "SQC_ICACHE_MISSES"],
}
FLUSH = "FillFunctor<float>"
COPY = "copyBuffer"
FUSED = "fused_kernel<"


def log(msg):
    print(f"[profile] {time.strftime('%H:%M:%S')} {msg}", flush=True)


def run(cmd, out_log, limit, kill_signal="TERM"):
    """One profiled process, under `timeout`; its output goes to out_log."""
    env = dict(os.environ, TMPDIR="/tmp")
    full = ["timeout", "-s", kill_signal, "-k", "10", str(limit)] + cmd
    with open(out_log, "w") as f:
        f.write("# " + " ".join(full) + "\n")
        f.flush()
        r = subprocess.run(full, cwd="/tmp", env=env, stdout=f, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise SystemExit(f"step failed ({r.returncode}): {' '.join(full)}; see {out_log}")


def find_db(d):
    dbs = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))
    if not dbs:
        raise SystemExit(f"no results database under {d}")
    return dbs[-1]


def bench_line(log_path):
    for line in reversed(open(log_path).read().splitlines()):
        if line.startswith("{") and '"metric"' in line:
            return json.loads(line)
    raise SystemExit(f"no bench line in {log_path}")


# ---- kernel trace ----

def timed_steps(db, n_steps, n_variants):
    """Dispatches of the timed rounds, cut into steps at the cache flushes:
    [(variant index, [(name, duration_ns, start, end), ...]), ...]."""
    c = sqlite3.connect(db)
    rows = c.execute("select name, duration, start, end from kernels order by start").fetchall()
    steps, cur = [], None
    for r in rows:
        if FLUSH in r[0]:
            cur = []
            steps.append(cur)
        elif cur is not None:
            cur.append(r)
    want = n_steps * n_variants
    if len(steps) < want:
        raise SystemExit(f"{len(steps)} flush-delimited steps in the trace, expected at least {want}")
    steps = steps[-want:]
    return [(i % n_variants, s) for i, s in enumerate(steps)]


def trace_table(db):
    c = sqlite3.connect(db)
    rows = c.execute("select name, total_calls, total_duration, average, percentage from top_kernels").fetchall()
    out = [f"{'calls':>6} {'total_us':>12} {'avg_us':>10} {'pct':>6}  kernel"]
    for name, calls, total, avg, pct in rows:
        name = name if len(name) <= 130 else name[:127] + "..."
        out.append(f"{calls:>6} {total:>12.1f} {avg:>10.2f} {pct:>6.2f}  {name}")
    return out


def summarize_trace(db, line, khash):
    # the bench's round order: fused, unfused sequence, plain GEMM, other gain placement,
    # the vendor library's plain product
    variants = ["fused"]
    if line.get("unfused_ms") is not None:
        variants.append("unfused")
    if line.get("plain_gemm_ms") is not None:
        variants.append("plain_gemm")
    other = [k for k in ("fused_in_loop_gain_ms", "fused_folded_gain_ms") if k in line]
    if other:
        variants.append(other[0][:-3])
    if line.get("vendor_gemm_ms") is not None:
        variants.append("vendor_gemm")
    steps = timed_steps(db, line["steps"], len(variants))
    per = collections.defaultdict(list)
    names = collections.defaultdict(collections.Counter)
    for v, disp in steps:
        per[v].append(sum(d for _, d, _, _ in disp) / 1e6)   # ms of kernel time in the step
        for n, *_ in disp:
            names[v][n] += 1
    fused_names = [n for n in names[0] if FUSED in n]
    if len(names[0]) != 1 or len(fused_names) != 1:
        raise SystemExit(f"the fused step should be one fused_kernel dispatch, found {dict(names[0])}")
    fused_name = fused_names[0]
    hdr = [
        f"# rocprofv3 kernel trace of bench.py: {bench.WORKLOAD_TEXT[line_workload(line)]}",
        f"# command: python3 profile_bench.py --out <dir> --workload {line_workload(line)}",
        f"#   which runs: rocprofv3 --kernel-trace --stats -d <dir> -o run -- python3 <repo>/bench.py "
        f"--workload {line_workload(line)} --no-cpu-baseline",
        f"# kernel source hash: {khash}",
        f"# headline (fused) kernel: {fused_name}",
        "# FillFunctor<float> is the 512 MiB cache flush before every step; the table's averages include the",
        "# warm-up rounds.",
        "",
    ]
    body = trace_table(db)
    tail = ["", f"# timed rounds: the last {line['steps']} rounds of {len(variants)} steps ({', '.join(variants)}),"
                " cut at the flushes"]
    rec = {}
    for i, v in enumerate(variants):
        ms = sorted(per[i])
        mean = sum(ms) / len(ms)
        med = ms[len(ms) // 2] if len(ms) % 2 else 0.5 * (ms[len(ms) // 2 - 1] + ms[len(ms) // 2])
        bench_stats = line[v + "_ms"]
        kinds = ", ".join(f"{n if len(n) < 70 else n[:67] + '...'} x{c // line['steps']}"
                          for n, c in names[i].items())
        tail.append(f"#   {v}: kernel time per step (trace) mean {mean:.4f} ms, median {med:.4f} ms "
                    f"(min {ms[0]:.4f}, max {ms[-1]:.4f}); bench events median {bench_stats['median']:.4f} ms, "
                    f"mean {bench_stats['mean']:.4f} ms")
        tail.append(f"#      kernels per step: {kinds}")
        rec[v] = {"trace_mean_ms": round(mean, 6), "trace_median_ms": round(med, 6),
                  "bench_median_ms": bench_stats["median"], "bench_mean_ms": bench_stats["mean"]}
    tail.append(f"# bench line of this run: value {line['value']} {line['unit']}, "
                f"speedup_vs_unfused {line.get('speedup_vs_unfused')}, tile {line['config'].get('tile')}")
    return "\n".join(hdr + body + tail) + "\n", fused_name, rec


def line_workload(line):
    text = line["config"]["workload"]
    for k, v in bench.WORKLOAD_TEXT.items():
        if text.startswith(v):
            return k
    raise SystemExit(f"unknown workload text {text!r}")


# ---- counters ----

def counters(db):
    """{kernel name: [{counter: value summed over instances, '_duration_ns': d}, ...]} per dispatch."""
    c = sqlite3.connect(db)
    q = ("select dispatch_id, kernel_name, counter_name, sum(value), avg(duration) from counters_collection "
         "group by dispatch_id, counter_name")
    per = collections.defaultdict(dict)
    names = {}
    for disp, kname, cname, val, dur in c.execute(q):
        per[disp][cname] = val
        per[disp]["_duration_ns"] = dur
        names[disp] = kname
    out = collections.defaultdict(list)
    for disp in sorted(per):
        out[names[disp]].append(per[disp])
    return out


def headline_dispatches(cnt, fused_name):
    if fused_name not in cnt:
        raise SystemExit(f"no dispatch of the headline kernel in the counter run: {fused_name}")
    return cnt[fused_name]


def avg(ds, counter):
    vals = [d[counter] for d in ds if counter in d]
    return sum(vals) / len(vals) if vals else None


def copy_scale(cnt, counter):
    copies = [d[counter] for n, ds in cnt.items() if COPY in n for d in ds if counter in d]
    if not copies:
        raise SystemExit(f"no calibration copy with {counter}")
    ref_kib = max(copies)
    return ref_kib, bench.COPY_BYTES / (ref_kib * 1024.0)


def profile(args, n):
    key = bench.WORKLOAD_KEY[n]
    khash = bench.kernel_source_hash()
    # absolute: the profiled processes run from /tmp.  The results databases
    # (large) go under --raw, the logs and the summaries under --out.
    out = os.path.join(os.path.abspath(args.raw), key)
    logs = os.path.join(os.path.abspath(args.out), key)
    summ = os.path.join(os.path.abspath(args.out), "summaries")
    for d in (out, logs, summ):
        os.makedirs(d, exist_ok=True)
    bench_py = os.path.join(ROOT, "bench.py")
    py = sys.executable or "python3"

    log(f"{key}: kernel trace")
    run(["rocprofv3", "--kernel-trace", "--stats", "-d", os.path.join(out, "kt"), "-o", "run", "--",
         py, bench_py, "--workload", str(n), "--no-cpu-baseline"], os.path.join(logs, "kt.log"), args.trace_limit)
    line = bench_line(os.path.join(logs, "kt.log"))
    text, fused_name, trace_rec = summarize_trace(find_db(os.path.join(out, "kt")), line, khash)
    with open(os.path.join(summ, f"{key}_kernel_trace.txt"), "w") as f:
        f.write(text)
    log(f"{key}: kernel trace summarised ({fused_name[:80]})")

    cnt = {}
    for name, ctrs in PASSES.items():
        log(f"{key}: counter pass {name}")
        run(["rocprofv3", "--pmc", *ctrs, "-d", os.path.join(out, name), "-o", "run", "--",
             py, bench_py, "--workload", str(n), "--no-cpu-baseline", "--no-unfused", "--copy-calibration",
             "--steps", "3", "--warmup", "2", "--warmup-seconds", "0.3"],
            os.path.join(logs, name + ".log"), args.counter_limit, kill_signal="KILL")
        cnt[name] = counters(find_db(os.path.join(out, name)))
        log(f"{key}: counter pass {name} done")

    cmd = f"python3 profile_bench.py --out <dir> --workload {n}"
    fetch_kib, fetch_scale = copy_scale(cnt["fetch"], "FETCH_SIZE")
    write_kib, write_scale = copy_scale(cnt["write"], "WRITE_SIZE")
    fd = headline_dispatches(cnt["fetch"], fused_name)
    wd = headline_dispatches(cnt["write"], fused_name)
    fetch_b = avg(fd, "FETCH_SIZE") * 1024.0 * fetch_scale
    write_b = avg(wd, "WRITE_SIZE") * 1024.0 * write_scale
    spec = __import__("workloads").get_config(n)
    traffic = {
        "workload": key,
        "kernel": fused_name,
        "kernel_source_hash": khash,
        "command": cmd,
        "counters": "rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE (KiB per dispatch, summed over the L2 "
                    "channels), each scaled by 256 MiB / (the counter for a plain 256 MiB device copy in the "
                    "same process); they count L2-to-fabric bytes (L2 misses, served by the Infinity Cache "
                    "or HBM), an upper bound on HBM bytes",
        "fetch": {"copy_counter_kib": fetch_kib, "scale": fetch_scale, "kernel_avg_kib": avg(fd, "FETCH_SIZE"),
                  "bytes": fetch_b, "dispatches": len(fd)},
        "write": {"copy_counter_kib": write_kib, "scale": write_scale, "kernel_avg_kib": avg(wd, "WRITE_SIZE"),
                  "bytes": write_b, "dispatches": len(wd)},
        "bytes_per_launch": int(round(fetch_b + write_b)),
        "algorithmic_bytes_per_launch": int(bench.algorithmic_bytes(spec)),
    }
    with open(os.path.join(summ, f"{key}_traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)

    a = headline_dispatches(cnt["sq_mfma_lds"], fused_name)
    b = headline_dispatches(cnt["sq_valu_wait"], fused_name)
    dur_ns = avg(a, "_duration_ns")
    cycles = avg(a, "GRBM_GUI_ACTIVE") / NUM_XCD          # per XCD: the shader clock cycles of the dispatch
    clock = cycles / dur_ns                                  # GHz
    mfma_busy = avg(a, "SQ_VALU_MFMA_BUSY_CYCLES")
    mops = avg(a, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    raw = {}
    ic = headline_dispatches(cnt["sqc_icache"], fused_name)
    for name, ds in (("sq_mfma_lds", a), ("sq_valu_wait", b), ("sqc_icache", ic)):
        for ctr in PASSES[name]:
            raw[f"{name}.{ctr}"] = avg(ds, ctr)
        raw[f"{name}.duration_us"] = avg(ds, "_duration_ns") / 1e3
    fused = {
        "dispatches": len(a),
        "duration_us": round(dur_ns / 1e3, 2),
        # GRBM_GUI_ACTIVE summed over the 8 XCDs: cycles per XCD over the duration
        "clock_ghz": round(clock, 4),
        # MFMA pipe busy, summed over the 1024 SIMDs, over the SIMD-cycles of the dispatch
        "mfma_busy_pct": round(100.0 * mfma_busy / (NUM_SIMD * cycles), 2),
        # cross-check: the bf16 MFMA ops counter (units of 512 flops) against the algorithmic 2MNK
        "mfma_mops_flops_over_2mnk": None if not mops else round(mops * 512.0 / float(spec.flops), 4),
        "achieved_tflops_in_counter_run": round(float(spec.flops) / (dur_ns * 1e-9) / 1e12, 1),
        # dense peak at that clock: 256 CUs x 4096 bf16 (256 fp32) flop per clock
        "peak_tflops_at_clock": round((256.0 if spec.ab_dtype == "f32" else 4096.0) * 256 * clock * 1e-3, 1),
        "valu_insts_per_wave": None if not raw["sq_valu_wait.SQ_WAVES"] else
        round(raw["sq_valu_wait.SQ_INSTS_VALU"] / raw["sq_valu_wait.SQ_WAVES"], 1),
        "lds_insts_per_wave": None if not raw["sq_valu_wait.SQ_WAVES"] else
        round(raw["sq_mfma_lds.SQ_INSTS_LDS"] / raw["sq_valu_wait.SQ_WAVES"], 1),
        # instruction cache: misses per request of the SQCs (each shared by a pair of CUs)
        "icache_miss_pct": None if not raw["sqc_icache.SQC_ICACHE_REQ"] else
        round(100.0 * raw["sqc_icache.SQC_ICACHE_MISSES"] / raw["sqc_icache.SQC_ICACHE_REQ"], 2),
    }
    rec = {
        "workload": key,
        "kernel": fused_name,
        "kernel_source_hash": khash,
        "command": cmd,
        "passes": {k: " ".join(v) for k, v in PASSES.items() if k.startswith("sq")},
        "note": "counter runs serialise dispatches; the headline kernel alone (bench.py --no-unfused), "
                "3 timed steps after a short warm-up. Raw values are per dispatch, summed over hardware "
                "instances; the LDS counters are reported as read and not cross-checked.",
        "fused": fused,
        "trace": trace_rec,
        "raw": raw,
    }
    with open(os.path.join(summ, f"{key}_counters.json"), "w") as f:
        json.dump(rec, f, indent=1)
    log(f"{key}: summaries written (clock {clock:.3f} GHz, MFMA busy {fused['mfma_busy_pct']}%, "
        f"traffic {traffic['bytes_per_launch'] / 1e6:.1f} MB)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", required=True, help="logs and summaries")
    ap.add_argument("--raw", default="/tmp/coda_profile_raw", help="rocprofv3 results databases")
    ap.add_argument("--workload", type=int, action="append", choices=sorted(bench.WORKLOAD_TEXT))
    ap.add_argument("--trace-limit", type=int, default=240, help="seconds for the kernel-trace run")
    ap.add_argument("--counter-limit", type=int, default=90, help="seconds for each counter pass")
    args = ap.parse_args()
    os.makedirs(args.out, exist_ok=True)
    for n in args.workload or sorted(bench.WORKLOAD_TEXT):
        profile(args, n)
    return 0


if __name__ == "__main__":
    sys.exit(main())
