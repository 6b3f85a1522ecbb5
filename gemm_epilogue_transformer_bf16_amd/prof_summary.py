"""Summarise a rocprofv3 results database (rocpd SQLite) as text.

  python -m gemm_epilogue_transformer_bf16_amd.prof_summary trace <results.db>
      per-kernel calls, total and average duration (us)
  python -m gemm_epilogue_transformer_bf16_amd.prof_summary pmc <results.db> [<results.db> ...]
      per-kernel average of each collected counter (summed over the hardware
      instances of one dispatch), plus the average dispatch duration
  python -m gemm_epilogue_transformer_bf16_amd.prof_summary traffic <fetch.db> <write.db> <kernel-substring> <copy-bytes>
      HBM bytes per launch of the kernel from FETCH_SIZE / WRITE_SIZE (KiB per
      dispatch), each scaled by bytes / counter of the plain device copy
      (__amd_rocclr_copyBuffer) of <copy-bytes> bytes in the same run; JSON
"""
from __future__ import annotations

import collections
import sqlite3
import sys


def short(name: str, width: int = 110) -> str:
    return name if len(name) <= width else name[: width - 3] + "..."


def trace(db: str) -> str:
    c = sqlite3.connect(db)
    rows = c.execute("select name, total_calls, total_duration, average, percentage from top_kernels").fetchall()
    # top_kernels reports durations in microseconds
    out = [f"{'calls':>6} {'total_us':>12} {'avg_us':>10} {'pct':>6}  kernel"]
    for name, calls, total, avg, pct in rows:
        out.append(f"{calls:>6} {total:>12.1f} {avg:>10.2f} {pct:>6.2f}  {short(name)}")
    return "\n".join(out)


def last_dispatches(db: str, kernel_substring: str, n: int) -> str:
    """Average duration (us) of the last n dispatches of the kernel: the timed
    steps of a run that starts with untimed warm-up steps."""
    c = sqlite3.connect(db)
    rows = c.execute("select name, duration from kernels order by start").fetchall()
    d = [dur for name, dur in rows if kernel_substring in name]
    if not d:
        return f"no dispatch of {kernel_substring!r}"
    tail = d[-n:]
    return (f"{len(tail)} last dispatches of {kernel_substring!r} (of {len(d)}): "
            f"avg {sum(tail) / len(tail) / 1000.0:.2f} us, min {min(tail) / 1000.0:.2f}, max {max(tail) / 1000.0:.2f}")


def pmc(dbs) -> str:
    per_kernel = collections.defaultdict(lambda: collections.defaultdict(list))
    durations = collections.defaultdict(dict)
    for db in dbs:
        c = sqlite3.connect(db)
        q = ("select dispatch_id, kernel_name, counter_name, sum(value), avg(duration) "
             "from counters_collection group by dispatch_id, counter_name")
        for disp, kname, cname, val, dur in c.execute(q):
            per_kernel[kname][cname].append(val)
            durations[kname][(db, disp)] = dur
    out = []
    for kname, counters in per_kernel.items():
        d = list(durations[kname].values())
        out.append(f"{short(kname)}")
        out.append(f"    dispatches={len(d)}  avg_duration_us={sum(d) / len(d) / 1000.0:.2f}")
        for cname, vals in sorted(counters.items()):
            out.append(f"    {cname:32s} avg={sum(vals) / len(vals):.6g}  (n={len(vals)})")
    return "\n".join(out)


def _counter_per_dispatch(db: str, counter: str):
    c = sqlite3.connect(db)
    q = ("select dispatch_id, kernel_name, sum(value) from counters_collection "
         "where counter_name = ? group by dispatch_id")
    return [(k, v) for _, k, v in c.execute(q, (counter,))]


def traffic(fetch_db: str, write_db: str, kernel: str, copy_bytes: int) -> dict:
    out = {}
    for counter, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        rows = _counter_per_dispatch(db, counter)
        copies = sorted(v for k, v in rows if "copyBuffer" in k)
        if not copies:
            raise SystemExit(f"no copy kernel in {db}")
        ref_kib = copies[-1]                       # the large calibration copy
        scale = copy_bytes / (ref_kib * 1024.0)
        vals = [v for k, v in rows if kernel in k]
        if not vals:
            raise SystemExit(f"no dispatch of {kernel!r} in {db}")
        avg_kib = sum(vals) / len(vals)
        out[counter] = {"copy_counter_kib": ref_kib, "scale": scale, "kernel_avg_kib": avg_kib,
                        "kernel_bytes": avg_kib * 1024.0 * scale, "dispatches": len(vals)}
    out["hbm_bytes_per_launch"] = out["FETCH_SIZE"]["kernel_bytes"] + out["WRITE_SIZE"]["kernel_bytes"]
    return out


def bench_profiles(out_dir: str, kt_db: str, fetch_db: str, write_db: str, command: str) -> None:
    """The two summaries kept for the LLaMA-7B gate/up bench: the kernel trace
    with a header naming the command and kernel sources, and the calibrated
    HBM traffic of the fused kernel."""
    import json
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    khash = bench.kernel_source_hash()
    header = [
        "# rocprofv3 kernel trace of bench.py (LLaMA-7B SwiGLU gate/up: M=4096, N=22016, K=4096)",
        f"# command: {command}",
        "#   (runs: rocprofv3 --kernel-trace --stats -- python3 bench.py --steps 10 --warmup 20 --no-cpu-baseline)",
        "# fused kernel: Cfg<256,256,2,4,fp32 operands=false,B[KxN]=true,norm=3 (RMS, gain folded into B),A[KxM]=false>;",
        "# the <..., 1, false> kernel is the same layer with the gain applied to A in the main loop (timed for",
        "# comparison), the <..., 0, false> kernel the plain GEMM of the unfused sequence, ew_kernel /",
        "# rownorm_kernel its other passes;",
        "# FillFunctor<float> is the 512 MiB cache flush between steps; averages include the warm-up steps.",
        f"# kernel source hash: {khash}",
    ]
    fused = "false, true, 3, false>"   # Cfg<..., fp32 operands, B stored [K x N], norm 3 (RMS, gain in B), A stored [K x M]>
    timed = "# timed steps: " + last_dispatches(kt_db, fused, 10)
    with open(os.path.join(out_dir, "fused_llama7b_gate_up_kernel_trace.txt"), "w") as f:
        f.write("\n".join(header) + "\n" + trace(kt_db) + "\n" + timed + "\n")
    t = traffic(fetch_db, write_db, fused, 256 << 20)
    spec_bytes = 2 * (4096 * 4096 + 4096 * 22016 + 4096 + 4096 * 11008)
    rec = {
        "kernel": "fused_kernel<Cfg<256, 256, 2, 4, bf16, B row-major [K x N], deferred RMS with the gain folded "
                  "into B>> on llama7b_swiglu_gate_up (M=4096, N=22016, K=4096)",
        "kernel_source_hash": khash,
        "command": command,
        "counters": "rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE (KiB per dispatch), each scaled by "
                    "256 MiB / (counter of a plain 256 MiB device copy in the same run)",
        "fetch": t["FETCH_SIZE"],
        "write": t["WRITE_SIZE"],
        "hbm_bytes_per_launch": int(round(t["hbm_bytes_per_launch"])),
        "algorithmic_bytes_per_launch": spec_bytes,
    }
    with open(os.path.join(out_dir, "fused_llama7b_gate_up_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)


def main(argv):
    if len(argv) >= 2 and argv[1] == "bench-profiles":
        bench_profiles(*argv[2:7])
        return 0
    if len(argv) < 3 or argv[1] not in ("trace", "pmc", "traffic"):
        print(__doc__)
        return 2
    if argv[1] == "trace":
        print(trace(argv[2]))
    elif argv[1] == "pmc":
        print(pmc(argv[2:]))
    else:
        import json
        print(json.dumps(traffic(argv[2], argv[3], argv[4], int(argv[5])), indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
