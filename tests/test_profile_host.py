"""Host-side checks of profile_bench.py (no GPU): the trace is cut into steps at
the cache flushes and the timed rounds are attributed to the right variant;
the counter tables are summed per dispatch; the copy calibration is the
largest copy."""
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _trace_db(path, rounds, variants):
    c = sqlite3.connect(path)
    c.execute("create table kernels (name text, duration integer, start integer, end integer)")
    t = 0

    def k(name, dur):
        nonlocal t
        c.execute("insert into kernels values (?, ?, ?, ?)", (name, dur, t, t + dur))
        t += dur + 10

    k("input_generation", 5)
    k("void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>, x>", 3)   # zeros()
    for r in range(rounds):
        for v in range(variants):
            k("void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>, x>", 50)
            if v == 1:   # the unfused sequence: three kernels
                k("rownorm_kernel", 100 + r)
                k("fused_kernel<Cfg<0>>", 1000 + r)
                k("ew_kernel", 200)
            else:
                k(f"fused_kernel<Cfg<{v + 1}>>", 700 + 10 * v + r)
    c.commit()
    c.close()


def test_timed_steps_cut_at_flushes(tmp_path):
    import profile_bench as pb
    db = str(tmp_path / "t.db")
    _trace_db(db, rounds=7, variants=3)
    steps = pb.timed_steps(db, 4, 3)
    assert [v for v, _ in steps] == [0, 1, 2] * 4
    # the last 4 rounds are rounds 3..6
    fused = [s for v, s in steps if v == 0]
    assert [d for (_, d, _, _), in fused] == [703, 704, 705, 706]
    unf = [s for v, s in steps if v == 1]
    assert all([n for n, *_ in s] == ["rownorm_kernel", "fused_kernel<Cfg<0>>", "ew_kernel"] for s in unf)
    assert sum(d for _, d, _, _ in unf[0]) == 103 + 1003 + 200


def test_timed_steps_too_few(tmp_path):
    import pytest

    import profile_bench as pb
    db = str(tmp_path / "t.db")
    _trace_db(db, rounds=2, variants=2)
    with pytest.raises(SystemExit):
        pb.timed_steps(db, 4, 2)


def _counter_db(path):
    c = sqlite3.connect(path)
    c.execute("create table counters_collection (dispatch_id integer, kernel_name text, counter_name text, "
              "value real, duration integer)")
    rows = []
    for disp, name, scale in ((1, "__amd_rocclr_copyBuffer", 1.0), (2, "__amd_rocclr_copyBuffer", 2.0),
                              (3, "fused_kernel<A>", 3.0), (4, "fused_kernel<A>", 5.0)):
        for inst in range(4):   # four hardware instances per dispatch
            rows.append((disp, name, "FETCH_SIZE", 1000.0 * scale / 4, 500))
    c.executemany("insert into counters_collection values (?, ?, ?, ?, ?)", rows)
    c.commit()
    c.close()


def test_counters_summed_per_dispatch_and_copy_scale(tmp_path):
    import bench
    import profile_bench as pb
    db = str(tmp_path / "c.db")
    _counter_db(db)
    cnt = pb.counters(db)
    assert [d["FETCH_SIZE"] for d in cnt["fused_kernel<A>"]] == [3000.0, 5000.0]
    assert pb.avg(cnt["fused_kernel<A>"], "FETCH_SIZE") == 4000.0
    ref, scale = pb.copy_scale(cnt, "FETCH_SIZE")
    assert ref == 2000.0 and scale == bench.COPY_BYTES / (2000.0 * 1024)


def test_summarize_trace_variants_and_bench_stats(tmp_path):
    import profile_bench as pb
    db = str(tmp_path / "t.db")
    _trace_db(db, rounds=6, variants=4)
    c = sqlite3.connect(db)
    c.execute("create table top_kernels (name text, total_calls integer, total_duration real, average real, "
              "percentage real)")
    c.execute("insert into top_kernels values ('fused_kernel<Cfg<1>>', 6, 4.2, 0.7, 50.0)")
    c.commit()
    c.close()
    st = {"median": 1.0, "mean": 1.0, "p10": 1.0, "p90": 1.0}
    line = {"steps": 3, "fused_ms": st, "unfused_ms": st, "plain_gemm_ms": st, "fused_in_loop_gain_ms": st,
            "value": 1.0, "unit": "TFLOP/s", "speedup_vs_unfused": 1.0,
            "config": {"workload": pb.bench.WORKLOAD_TEXT[2], "tile": 1}}
    text, fused_name, rec = pb.summarize_trace(db, line, "0" * 16)
    assert fused_name == "fused_kernel<Cfg<1>>"
    assert set(rec) == {"fused", "unfused", "plain_gemm", "fused_in_loop_gain"}
    # the last three rounds: fused durations 703, 704, 705 ns
    assert abs(rec["fused"]["trace_mean_ms"] - 704e-6) < 1e-9


def test_summarize_trace_with_vendor_leg(tmp_path):
    import profile_bench as pb
    db = str(tmp_path / "t.db")
    _trace_db(db, rounds=5, variants=5)
    c = sqlite3.connect(db)
    c.execute("create table top_kernels (name text, total_calls integer, total_duration real, average real, "
              "percentage real)")
    c.commit()
    c.close()
    st = {"median": 1.0, "mean": 1.0, "p10": 1.0, "p90": 1.0}
    line = {"steps": 2, "fused_ms": st, "unfused_ms": st, "plain_gemm_ms": st, "fused_folded_gain_ms": st,
            "vendor_gemm_ms": st, "value": 1.0, "unit": "TFLOP/s", "speedup_vs_unfused": 1.0,
            "config": {"workload": pb.bench.WORKLOAD_TEXT[4], "tile": 3}}
    text, fused_name, rec = pb.summarize_trace(db, line, "0" * 16)
    assert list(rec) == ["fused", "unfused", "plain_gemm", "fused_folded_gain", "vendor_gemm"]
    # the vendor leg is the fifth step of each round: rounds 3 and 4 of variant 4
    assert abs(rec["vendor_gemm"]["trace_mean_ms"] - 743.5e-6) <= 0.5e-6   # rounded to 1 ns
    assert "vendor_gemm" in text
