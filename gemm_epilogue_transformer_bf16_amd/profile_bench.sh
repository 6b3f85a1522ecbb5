#!/bin/bash
# Profiles bench.py with rocprofv3 and writes text summaries under $OUT:
#   kernel trace + per-kernel duration stats, then FETCH_SIZE and WRITE_SIZE
#   counter passes (one counter group per run), calibrated against a plain
#   256 MiB device copy done in the same process.
# Usage (repo root): bash gemm_epilogue_transformer_bf16_amd/profile_bench.sh <out-dir>
set -o pipefail
OUT=$(mkdir -p "${1:?out dir}" && cd "$1" && pwd)
R=$(cd "$(dirname "$0")/.." && pwd)
mkdir -p "$OUT"
cd /tmp && export TMPDIR=/tmp
timeout -k 10 300 rocprofv3 --kernel-trace --stats -d "$OUT/kt" -o bench -- \
  python3 "$R/bench.py" --steps 10 --warmup 20 --no-cpu-baseline > "$OUT/bench_kt.log" 2>&1 || exit 1
echo "kernel trace done"
timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE -d "$OUT/fetch" -o p -- \
  python3 "$R/bench.py" --steps 3 --warmup 1 --no-cpu-baseline --no-unfused --copy-calibration > "$OUT/fetch.log" 2>&1 || exit 1
echo "fetch pass done"
timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE -d "$OUT/write" -o p -- \
  python3 "$R/bench.py" --steps 3 --warmup 1 --no-cpu-baseline --no-unfused --copy-calibration > "$OUT/write.log" 2>&1 || exit 1
echo "write pass done"
cd "$R"
python3 -m gemm_epilogue_transformer_bf16_amd.prof_summary trace "$OUT"/kt/*.db > "$OUT/trace.txt"
python3 -m gemm_epilogue_transformer_bf16_amd.prof_summary traffic "$OUT"/fetch/*.db "$OUT"/write/*.db "false, true, 3, false>" 268435456 > "$OUT/traffic.json"
python3 -m gemm_epilogue_transformer_bf16_amd.prof_summary bench-profiles "$OUT" "$(ls "$OUT"/kt/*.db)" \
  "$(ls "$OUT"/fetch/*.db)" "$(ls "$OUT"/write/*.db)" "bash gemm_epilogue_transformer_bf16_amd/profile_bench.sh <out-dir>"
echo "summaries done"
