"""Benchmark of the fused GEMM + epilogue path on one MI355X.

One step = one fused call (operand staging, in-loop gain and sum of squares,
MFMA main loop, ordered epilogue, one store of D) on the LLaMA-7B-shaped
SwiGLU gate/up layer: M = 4096 tokens, K = 4096, [W_gate | W_up] column
interleaved, N = 2 x 11008, deferred RMSNorm ((x * gamma) @ W in the main loop,
the per-row 1/rms in the epilogue) then SiLU(gate) * up, bf16 storage and fp32
accumulation.  Inputs are seeded synthetic tensors with the layer's shapes and
value distributions, resident in HBM before timing.  ``--workload`` times
another of the synthetic transformer layers instead.

Timing: the fused call, the in-run unfused HIP sequence (same main loop, one
kernel per operator, bf16 intermediates) and, for norm layers, the fused call
with the gain folded into a copy of the weights run round-robin, one step of
each per round, each step preceded by a cache flush and bracketed by HIP
events on the stream the library launches on.  The warm-up lasts at least
``--warmup`` rounds and ``--warmup-seconds`` of wall time, so the GPU clock has
settled whatever the round count.  Times are medians over the timed rounds
(p10 / p90 beside them).

Prints one JSON line: fused TFLOP/s (2 M N K / median kernel time), the share
of the bf16 dense MFMA peak (and of the peak at the shader clock the committed
counter run measured under the same kernel sources), the speedup over the
unfused sequence, the roofline object and the CPU-oracle baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0        # MI355X published dense bf16 MFMA peak
PEAK_F32_TFLOPS = 157.3          # MI355X published fp32 matrix peak
PEAK_HBM_GBPS = 8000.0
WORKLOAD_INDEX = 4               # LLaMA-7B SwiGLU gate/up
WORKLOAD_TEXT = {
    1: "tiny forward layer, fp32: deferred RMSNorm + bias + GELU_tanh + residual, M=N=K=256",
    2: "gpt2s_mlp_up: deferred RMSNorm + bias + GELU_tanh, M=8192 tokens, K=768, N=3072, bf16 in/out",
    3: "bertl_mlp_down: bias + residual + row sum and sum of squares, M=8192, K=4096, N=1024, bf16 in/out",
    4: "llama7b_swiglu_gate_up: deferred RMSNorm + SwiGLU(gate,up), M=4096 tokens, K=4096, "
       "N=2x11008 column-interleaved, bf16 in/out, fp32 accumulate",
    5: "gpt2m_mlp_bwd_act: dH = dY W2^T times GELU_tanh'(P) + row sum, M=8192, K=1024, N=4096, bf16 in/out",
    6: "gpt2s_mlp_up_layernorm: deferred LayerNorm + bias + GELU_tanh, M=8192 tokens, K=768, N=3072, bf16 in/out",
}


def algorithmic_bytes(spec) -> float:
    """One read of every input tensor, one write of D and of the reduction outputs."""
    size = {"bf16": 2, "f32": 4}
    b = sum(float(np.prod(t.shape)) * size[t.dtype] for t in spec.tensors)
    b += float(spec.M) * spec.out_width * size[spec.d_dtype]
    b += sum(float(np.prod(shape)) * 4 for _, shape in spec.outputs)
    return b
FLUSH_BYTES = 512 << 20          # larger than L2 (8 x 4 MB) plus the 256 MB Infinity Cache
COPY_BYTES = 256 << 20           # plain copy used to calibrate the HBM traffic counters


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gemm_epilogue_transformer_bf16_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def _profile_record(workload: str, kind: str):
    path = os.path.join(ROOT, "profiles", f"{workload}_{kind}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        return json.load(f)


def load_traffic(workload: str, kernel_hash: str):
    """L2-to-fabric bytes per launch of the fused kernel (FETCH_SIZE + WRITE_SIZE,
    each calibrated against a plain device copy) from the committed rocprofv3
    counter runs of this workload, if they were taken on the current kernel
    sources."""
    rec = _profile_record(workload, "traffic")
    if not rec or rec.get("kernel_source_hash") != kernel_hash:
        return None
    return rec.get("bytes_per_launch")


def load_counter_clock(workload: str, kernel_hash: str):
    """Shader clock (GHz) of the fused kernel from the committed counter run:
    GRBM_GUI_ACTIVE cycles (per XCD) over the dispatch duration."""
    return load_counter_field(workload, kernel_hash, "clock_ghz")


def load_counter_field(workload: str, kernel_hash: str, field: str):
    """A derived figure of the fused kernel from the committed counter run of
    this workload (clock_ghz, mfma_busy_pct), if it was taken on the current
    kernel sources."""
    rec = _profile_record(workload, "counters")
    if not rec or rec.get("kernel_source_hash") != kernel_hash:
        return None
    return rec.get("fused", {}).get(field)


def cpu_baseline(spec, inputs, budget_s: float = 10.0):
    """The fp64 oracle on a bounded row sample of the same workload."""
    import contextlib

    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:       # pragma: no cover
        threadpool_info = threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    ctx = threadpool_limits(limits=cores) if threadpool_limits else contextlib.nullcontext()
    with ctx:
        threads = cores
        if threadpool_info:
            info = threadpool_info()
            if info:
                threads = max(i.get("num_threads", cores) for i in info)
        rows_done = 0
        elapsed = 0.0
        chunk = 64
        order = np.random.default_rng(0).permutation(spec.M)
        oracle.run_workload(spec, inputs, order[:8])   # warm-up
        while elapsed < budget_s and rows_done < spec.M:
            rows = order[rows_done:rows_done + chunk]
            t0 = time.perf_counter()
            oracle.run_workload(spec, inputs, rows)
            elapsed += time.perf_counter() - t0
            rows_done += len(rows)
            chunk = min(chunk * 2, 1024)
    flops = 2.0 * rows_done * spec.N * spec.K
    return {
        "value": round(flops / elapsed / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{rows_done} of {spec.M} rows of the same layer (fp64 numpy: "
                  f"{', '.join(op for op, _ in spec.program)} around the matmul), {elapsed:.1f} s",
    }


class Timer:
    """Times C-ABI launch functions round-robin: per round one step of each, every
    step preceded by a cache flush (a 512 MiB fill, unless --no-flush) and
    bracketed by HIP events on torch's current stream, the stream the binding
    launches on.  The warm-up runs at least ``warmup`` rounds and
    ``warmup_seconds`` of wall time; then exactly ``steps`` rounds are timed
    between two device synchronisations."""

    def __init__(self, args):
        import torch
        self.args = args
        self.flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        self.wall_s = None

    def _step(self, fn):
        import torch
        from gemm_epilogue_transformer_bf16_amd import coda
        if not self.args.no_flush:
            self.flush.zero_()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        coda.check(fn(), "launch")
        s1.record()
        return s0, s1

    def run(self, fns):
        """fns: {name: launch function}; returns {name: per-step times in ms}."""
        import torch
        args = self.args
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        rounds = 0
        while rounds < args.warmup or time.perf_counter() - t0 < args.warmup_seconds:
            for fn in fns.values():
                self._step(fn)
            rounds += 1
            if rounds % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        evs = {name: [] for name in fns}
        for _ in range(args.steps):
            for name, fn in fns.items():
                evs[name].append(self._step(fn))
        torch.cuda.synchronize()
        self.wall_s = time.perf_counter() - t1
        self.warmup_rounds = rounds
        self.warmup_s = t1 - t0
        return {name: np.array([a.elapsed_time(b) for a, b in e]) for name, e in evs.items()}


def stats(ms):
    return {"median": round(float(np.median(ms)), 4), "mean": round(float(np.mean(ms)), 4),
            "p10": round(float(np.percentile(ms, 10)), 4), "p90": round(float(np.percentile(ms, 90)), 4)}


def result_line(args, timer, flops, fused_ms, unfused_ms, config, peak, alg_bytes, cpu, traffic=None,
                counter_clock=None, extra=None):
    """The JSON line: value = flops / median fused time."""
    ms = float(np.median(fused_ms))
    tflops = flops / (ms * 1e-3) / 1e12
    umed = None if unfused_ms is None else float(np.median(unfused_ms))
    line = {
        "metric": "fused GEMM+epilogue TFLOP/s, % bf16 MFMA peak; speedup vs unfused HIP",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if peak == PEAK_F32_TFLOPS else "bf16",
        "data": "synthetic",
        "config": config,
        "pct_peak": round(100.0 * tflops / peak, 2),
        "fused_ms": stats(fused_ms),
        "unfused_ms": None if unfused_ms is None else stats(unfused_ms),
        "unfused_ms_per_step": None if umed is None else round(umed, 4),
        "speedup_vs_unfused": None if umed is None else round(umed / ms, 3),
        "effective_GBps": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
        # the shader clock under this kernel (GRBM_GUI_ACTIVE cycles over the
        # dispatch time, from the committed counter run of the same sources) and
        # the dense peak at that clock: 256 CUs x 4096 bf16 flop per clock
        # (x 256 for fp32)
        "clock_ghz_counters": counter_clock,
        "pct_peak_at_measured_clock": None if not counter_clock else round(
            100.0 * tflops / ((4096.0 if peak != PEAK_F32_TFLOPS else 256.0) * 256 * counter_clock * 1e-3), 2),
        "timing": {"warmup_rounds": timer.warmup_rounds, "warmup_s": round(timer.warmup_s, 3),
                   "timed_rounds_wall_s": round(timer.wall_s, 4), "interleaved": True,
                   "cache_flush_between_steps": not args.no_flush},
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4),
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
        "kernel_source_hash": kernel_source_hash(),
    }
    if extra:
        line.update(extra)
    return line


def bench_weight_grad(args):
    """dW_acc += X^T dY for the GPT-2-small MLP up-projection (X [8192 tokens x
    768], dY [8192 x 3072], dW [768 x 3072], K = 8192 tokens): A stored [K x M]
    and the accumulation into the gradient buffer fused as an in-place ADD_MAT."""
    import oracle
    import workloads as w
    from gemm_epilogue_transformer_bf16_amd import coda, runner

    T, Fi, Fo = 8192, 768, 3072
    rng = np.random.default_rng(2001)
    x = w.bf16_bits_from_f64(rng.standard_normal((T, Fi)))
    dy = w.bf16_bits_from_f64(rng.standard_normal((T, Fo)) / np.sqrt(Fo))
    acc = w.bf16_bits_from_f64(0.01 * rng.standard_normal((Fi, Fo)))
    to_dev = lambda b: runner.storage_to_tensor(b, "bf16")
    X, dY, ACC = to_dev(x), to_dev(dy), to_dev(acc)
    call = runner.Call(X, dY, [("add_mat", {"mat": ACC, "beta": 1.0})], "KN", a_layout="KM", D=ACC,
                       tile=args.tile)
    timer = Timer(args)
    fns = {"fused": call.fused}
    if not args.no_unfused:
        fns["unfused"] = call.unfused
    print("[bench] weight gradient: fused and unfused, interleaved", file=sys.stderr, flush=True)
    t = timer.run(fns)
    flops = 2.0 * T * Fi * Fo
    alg_bytes = 2.0 * (T * Fi + T * Fo + 2 * Fi * Fo)   # X, dY, the accumulator read and written
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        xs, dys, accs = (w.bf16_bits_to_f64(b) for b in (x, dy, acc))
        rows = np.random.default_rng(0).permutation(Fi)[:192]
        t0 = time.perf_counter()
        oracle.forward(xs[:, rows].T, dys, [("add_mat", {"mat": accs[rows], "beta": 1.0})], "KN")
        el = time.perf_counter() - t0
        cpu = {"value": round(2.0 * T * len(rows) * Fo / el / 1e12, 5), "unit": "TFLOP/s",
               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"{len(rows)} of {Fi} rows of dW (fp64 numpy: X^T dY + accumulator), {el:.1f} s"}
    config = {"workload": "gpt2s_mlp_up weight gradient: dW_acc += X^T dY, X [8192 tokens x 768], "
                          "dY [8192 x 3072], A stored [K x M], in-place accumulation, bf16",
              "M": Fi, "N": Fo, "K": T, "tile": coda.coda_selected_tile(Fi, Fo, T, call.desc)}
    line = result_line(args, timer, flops, t["fused"], t.get("unfused"), config, PEAK_BF16_TFLOPS, alg_bytes, cpu)
    print(json.dumps(line), flush=True)


def bench_rms_backward(args):
    """The RMS norm's backward through the LLaMA-7B gate/up projection:
    dX = RMS_BWD(dP W^T) with dgamma = RMS_DGAMMA(dP W^T) in the same epilogue;
    dP = d[gate|up] [4096 tokens x 22016], W [4096 x 22016] read as the [N x K]
    operand (N = 4096 features, K = 22016), x [4096 x 4096] the norm's input.
    The row statistics (sum of squares of x, and t = sum dP * P, which the GEMM
    producing dP would reduce) are given; they are prepared before timing."""
    import torch
    import oracle
    import workloads as w
    from gemm_epilogue_transformer_bf16_amd import coda, runner

    T, F, Np, eps = 4096, 4096, 2 * 11008, 1e-6
    rng = np.random.default_rng(2002)
    xb = w.bf16_bits_from_f64(rng.standard_normal((T, F)))
    gb = w.bf16_bits_from_f64(1 + 0.1 * rng.standard_normal(F))
    wb = w.bf16_bits_from_f64(rng.standard_normal((F, Np)) / np.sqrt(F))
    dpb = w.bf16_bits_from_f64(rng.standard_normal((T, Np)) / np.sqrt(Np))
    to_dev = lambda b: runner.storage_to_tensor(b, "bf16")
    X, G, W, dP = to_dev(xb), to_dev(gb), to_dev(wb), to_dev(dpb)
    stats_t = torch.empty((T, 2), dtype=torch.float32, device="cuda")
    stats_t[:, 0] = X.float().pow(2).sum(dim=1)
    stats_t[:, 1] = torch.from_numpy(rng.standard_normal(T).astype(np.float32)).cuda()
    dg = torch.zeros((F, 1), dtype=torch.float32, device="cuda")
    ops = [("rms_dgamma", {"x": X, "eps": eps, "stats": stats_t, "sumsq_col": 0, "out": dg, "col": 0}),
           ("rms_bwd", {"x": X, "gamma": G, "eps": eps, "stats": stats_t, "sumsq_col": 0, "t_col": 1})]
    call = runner.Call(dP, W, ops, "NK", tile=args.tile)
    timer = Timer(args)
    fns = {"fused": call.fused}
    if not args.no_unfused:
        fns["unfused"] = call.unfused
    print("[bench] rms backward: fused and unfused, interleaved", file=sys.stderr, flush=True)
    t = timer.run(fns)
    flops = 2.0 * T * F * Np
    alg_bytes = 2.0 * (T * Np + F * Np + 2 * T * F)   # dP, W, x read; dX written
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        rows = np.random.default_rng(0).permutation(T)[:512]
        x64, g64, w64, dp64 = (w.bf16_bits_to_f64(b) for b in (xb, gb, wb, dpb))
        t0 = time.perf_counter()
        oracle.forward(dp64[rows], w64.T, [("rms_dgamma", {"x": x64[rows], "eps": eps}),
                                           ("rms_bwd", {"x": x64[rows], "gamma": g64, "eps": eps})], "KN")
        el = time.perf_counter() - t0
        cpu = {"value": round(2.0 * len(rows) * F * Np / el / 1e12, 5), "unit": "TFLOP/s",
               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"{len(rows)} of {T} rows of dX (fp64 numpy: dP W^T, the norm's backward), {el:.1f} s"}
    config = {"workload": "llama7b RMSNorm backward through the gate/up projection: dX = RMS_BWD(dP W^T) "
                          "and dgamma = RMS_DGAMMA(dP W^T), dP [4096 tokens x 22016], W [4096 x 22016], "
                          "row statistics given, bf16",
              "M": T, "N": F, "K": Np, "tile": coda.coda_selected_tile(T, F, Np, call.desc)}
    line = result_line(args, timer, flops, t["fused"], t.get("unfused"), config, PEAK_BF16_TFLOPS, alg_bytes, cpu)
    print(json.dumps(line), flush=True)


WORKLOAD_KEY = {1: "tiny_fwd", 2: "gpt2s_mlp_up", 3: "bertl_mlp_down", 4: "llama7b_gate_up",
                5: "gpt2m_mlp_bwd", 6: "gpt2s_mlp_up_layernorm"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed rounds (one step of each variant per round)")
    ap.add_argument("--warmup", type=int, default=10, help="untimed rounds first (at least)")
    ap.add_argument("--warmup-seconds", type=float, default=0.6,
                    help="the warm-up lasts at least this long: the clock needs a few hundred ms to settle")
    ap.add_argument("--tile", type=int, default=0, help="force a tile configuration (0 = automatic)")
    ap.add_argument("--workload", type=int, default=WORKLOAD_INDEX, choices=sorted(WORKLOAD_TEXT),
                    help="synthetic layer to time (default: the LLaMA-7B gate/up layer)")
    ap.add_argument("--no-flush", action="store_true", help="do not evict L2 / Infinity Cache between steps")
    ap.add_argument("--bias-grad", action="store_true",
                    help="GPT-2-medium backward layer (workload 5) with the bias gradient: a column sum of dH "
                         "appended to its epilogue")
    ap.add_argument("--given-row-sumsq", action="store_true",
                    help="RMSNorm / LayerNorm layers: the row sums of squares (and sums) of A are given (as the "
                         "previous layer's ROW_SUMSQ / ROW_SUM outputs provide them in a chain of layers; computed "
                         "here before timing) and the gain is folded, so the main loop is the plain GEMM")
    ap.add_argument("--weight-grad", action="store_true",
                    help="the GPT-2-small MLP up-projection's weight gradient, dW_acc += X^T dY, instead")
    ap.add_argument("--rms-backward", action="store_true",
                    help="time the RMS norm's backward through the LLaMA-7B gate/up projection instead")
    ap.add_argument("--fold-gain", action="store_true",
                    help="headline = the RMSNorm / LayerNorm gain folded into a copy of the weights once "
                         "(coda_fold_gain, outside the timed region) instead of applied to A in the main loop; "
                         "the other placement is timed beside it either way")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unfused", action="store_true")
    ap.add_argument("--no-vendor", action="store_true",
                    help="skip the torch.matmul timing of the plain product (reported for context)")
    ap.add_argument("--all", action="store_true",
                    help="every synthetic layer in turn: one line with each layer's fused, unfused and plain-GEMM "
                         "medians, speedups beside the ceilings, and their geometric mean")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device copy three times (reference for traffic counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the fused GEMM + epilogue path runs on one GPU.", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.rms_backward:
        bench_rms_backward(args)
        return
    if args.weight_grad:
        bench_weight_grad(args)
        return

    if args.all:
        bench_all(args)
        return
    line = measure_workload(args, args.workload)
    print(json.dumps(line), flush=True)


def measure_workload(args, workload: int, cpu_baseline_on: bool = True):
    """Times one synthetic layer (fused, the unfused sequence, the plain GEMM
    with an empty list and, for norm layers, the other gain placement,
    round-robin) and returns the JSON line as a dict."""
    import torch
    import workloads as w
    from gemm_epilogue_transformer_bf16_amd import coda, runner
    TORCH_DT_OF = runner.TORCH_DT

    spec = w.get_config(workload)
    if args.bias_grad:
        import dataclasses
        if workload != 5:
            print("--bias-grad applies to the backward layer (--workload 5)", file=sys.stderr)
            sys.exit(2)
        spec = dataclasses.replace(spec, program=spec.program + (("col_sum", {"out": "db", "col": 0}),),
                                   outputs=spec.outputs + (("db", (spec.out_width, 1)),))
    print(f"[bench] generating {spec.name} inputs", file=sys.stderr, flush=True)
    inputs = w.make_inputs(spec)
    has_rms = any(op == "rms_rowscale" for op, _ in spec.program)
    has_norm = has_rms or any(op == "ln_rowscale" for op, _ in spec.program)
    fold = has_norm and (args.fold_gain or args.given_row_sumsq)
    call = runner.WorkloadCall(spec, inputs, tile=args.tile, fold_gain=fold)
    tensors = call.tensors
    if args.given_row_sumsq:
        if not has_norm:
            print("--given-row-sumsq applies to layers with an RMSNorm or LayerNorm", file=sys.stderr)
            sys.exit(2)
        # setup outside the timed region: the row sums and sums of squares a
        # previous layer's ROW_SUM / ROW_SUMSQ epilogue would have written
        A = tensors[spec.a_name]
        row_stats = torch.stack([A.float().sum(dim=1), (A.float() * A.float()).sum(dim=1)], dim=1).contiguous()
        prog = [(n, dict(a)) for n, a in call.ops]
        prog[0][1].update({"row_ss": row_stats, "row_ss_col": 1, "row_s_col": 0})
        call = runner.Call(A, call.B, prog, spec.b_layout, d_dtype=TORCH_DT_OF[spec.d_dtype], tile=args.tile)
    torch.cuda.synchronize()
    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    tile_used = coda.coda_selected_tile(spec.M, spec.N, spec.K, call.desc)

    fns = {"fused": call.fused}
    other = plain = None
    if not args.no_unfused:
        fns["unfused"] = call.unfused
        # the same main loop with an empty list: the fused kernel's time if its
        # epilogue were free, so unfused / plain is the most fusion can gain here
        plain = runner.Call(tensors[spec.a_name], tensors[spec.b_name], [], spec.b_layout,
                            d_dtype=TORCH_DT_OF[spec.d_dtype], tile=args.tile, M=spec.M, N=spec.N, K=spec.K)
        fns["plain"] = plain.fused
        if has_norm and not args.given_row_sumsq:
            # the other placement of the norm's gain, for comparison (not the headline)
            other = runner.WorkloadCall(spec, inputs, tile=args.tile, fold_gain=not fold)
            fns["other"] = other.fused
    if not args.no_unfused and not args.no_vendor:
        # context only: the vendor library's plain product of the same operands
        # (torch.matmul; B stored [N x K] is given to it transposed once, here)
        va = tensors[spec.a_name]
        vb = tensors[spec.b_name] if spec.b_layout == "KN" else tensors[spec.b_name].t().contiguous()
        vd = torch.empty((spec.M, spec.N), dtype=va.dtype, device=va.device)

        def vendor_gemm():
            torch.matmul(va, vb, out=vd)
            return 0
        fns["vendor"] = vendor_gemm
    timer = Timer(args)
    print(f"[bench] {', '.join(fns)}: warm-up >= {args.warmup} rounds and {args.warmup_seconds} s, "
          f"then {args.steps} timed rounds", file=sys.stderr, flush=True)
    t = timer.run(fns)

    flops = float(spec.flops)
    peak = PEAK_F32_TFLOPS if spec.ab_dtype == "f32" else PEAK_BF16_TFLOPS
    alg_bytes = algorithmic_bytes(spec)
    khash = kernel_source_hash()
    key = WORKLOAD_KEY[workload]
    plain_variant = not (args.bias_grad or args.given_row_sumsq or args.fold_gain or args.tile or args.no_flush)
    traffic = load_traffic(key, khash) if plain_variant else None
    counter_clock = load_counter_clock(key, khash) if plain_variant else None
    mfma_busy = load_counter_field(key, khash, "mfma_busy_pct") if plain_variant else None

    cpu = None
    if cpu_baseline_on and not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(spec, inputs)

    config = {
        "workload": WORKLOAD_TEXT[workload] + (" + bias gradient (column sum of dH)" if args.bias_grad else ""),
        "M": spec.M, "N": spec.N, "K": spec.K,
        "gain": ("folded into a copy of the weights" if fold else "applied to A in the main loop")
                if has_norm else None,
        "row_sumsq_given": bool(args.given_row_sumsq),
        "tile": tile_used,
    }
    # MFMA pipe busy share of the SIMD-cycles in the committed counter run of
    # the same sources (the headline kernel alone, counters serialise dispatches)
    extra = {"mfma_busy_pct_counters": mfma_busy}
    if plain is not None:
        pmed, fmed, umed = (float(np.median(t[k])) for k in ("plain", "fused", "unfused"))
        extra["plain_gemm_ms"] = stats(t["plain"])
        extra["fused_over_plain"] = round(fmed / pmed, 3)
        extra["unfused_over_plain"] = round(umed / pmed, 3)
    if other is not None:
        extra[("fused_in_loop_gain_ms" if fold else "fused_folded_gain_ms")] = stats(t["other"])
    if "vendor" in t:
        extra["vendor_gemm_ms"] = stats(t["vendor"])
        extra["plain_over_vendor"] = round(float(np.median(t["plain"])) / float(np.median(t["vendor"])), 3)
        extra["vendor_gemm"] = "torch.matmul, the plain product only (context, not a baseline of the speedup)"
    return result_line(args, timer, flops, t["fused"], t.get("unfused"), config, peak, alg_bytes, cpu,
                       traffic=traffic, counter_clock=counter_clock, extra=extra)


# the per-layer speedup ceilings of fusion for the same main loop, computed from
# the unfused sequence's extra HBM passes (at 8 and at 5 TB/s) over the GEMM at
# 70% of the bf16 dense peak
CEILING = {2: (2.29, 3.06), 3: (1.27, 1.43), 4: (1.13, 1.20), 5: (1.65, 2.03)}


def bench_all(args):
    """Every synthetic layer in turn (fused, unfused, plain GEMM), one JSON
    line: each layer's medians and speedup beside the ceilings, and the
    geometric mean of the speedups over the bf16 layers."""
    if args.no_unfused:
        print("--all compares fused and unfused: drop --no-unfused", file=sys.stderr)
        sys.exit(2)
    rows = []
    for wl in sorted(WORKLOAD_TEXT):
        line = measure_workload(args, wl, cpu_baseline_on=False)
        rows.append({
            "workload": WORKLOAD_KEY[wl], "tile": line["config"]["tile"],
            "fused_ms": line["fused_ms"]["median"], "unfused_ms": line["unfused_ms"]["median"],
            "plain_gemm_ms": line["plain_gemm_ms"]["median"], "speedup_vs_unfused": line["speedup_vs_unfused"],
            "unfused_over_plain": line["unfused_over_plain"], "fused_over_plain": line["fused_over_plain"],
            "tflops": line["value"], "pct_peak": line["pct_peak"],
            "ceiling_at_8_and_5_TBps": CEILING.get(wl),
            "fused_p10_p90": [line["fused_ms"]["p10"], line["fused_ms"]["p90"]],
            "vendor_gemm_ms": line.get("vendor_gemm_ms", {}).get("median"),
        })
        print(f"[bench] {WORKLOAD_KEY[wl]}: fused {rows[-1]['fused_ms']} ms, unfused {rows[-1]['unfused_ms']} ms, "
              f"plain {rows[-1]['plain_gemm_ms']} ms", file=sys.stderr, flush=True)
    bf = [r["speedup_vs_unfused"] for r in rows if r["workload"] != WORKLOAD_KEY[1]]
    geo = float(np.exp(np.mean(np.log(bf))))
    out = {
        "metric": "fused vs unfused speedup, geometric mean over the bf16 synthetic layers",
        "value": round(geo, 3), "unit": "x", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": True, "data": "synthetic", "per_workload": rows,
        "geomean_unfused_over_plain": round(float(np.exp(np.mean(np.log(
            [r["unfused_over_plain"] for r in rows if r["workload"] != WORKLOAD_KEY[1]])))), 3),
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
