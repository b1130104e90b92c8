#!/bin/bash
# Kernel-trace and HBM-counter runs of bench.py for the profiles/ summaries.
# usage (on the GPU machine, from the repository root):
#   bench_probe/collect_counters.sh OUT tag "bench args" [tag "bench args"]...
# then, anywhere:  python bench.py --reduce-counters OUT
# Per workload: one rocprofv3 --kernel-trace --stats run, and one --pmc pass
# each for FETCH_SIZE and WRITE_SIZE (every pass ends with a plain 1 GiB
# device copy that calibrates the counters).  A profiler that exits non-zero
# after the program's result line was printed is reported and its complete
# results are kept; any other failure stops the script.
OUT=$(realpath -m "$1"); shift
R=$(cd "$(dirname "$0")/.." && pwd)
cd /tmp && export TMPDIR=/tmp
while [ $# -ge 2 ]; do
  tag=$1; args=$2; shift 2
  D=$OUT/$tag
  mkdir -p "$D"
  echo "$args" > "$D/args.txt"
  echo "[counters] $tag kernel trace ($args)"
  timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv -d "$D/kt" -o run -- \
    python3 "$R/bench.py" --steps 50 --warmup 5 --no-cpu-baseline $args > "$D/kt.json" 2> "$D/kt.err"
  rc=$?
  if [ $rc -ne 0 ]; then
    if [ $rc -eq 124 ] || [ $rc -eq 137 ] || ! grep -q metric "$D/kt.json"; then
      echo "[counters] $tag kernel trace failed (rc $rc)"; tail -5 "$D/kt.err"; exit $rc
    fi
    echo "[counters] $tag kernel trace: profiler rc $rc after a complete run"
  fi
  for c in FETCH_SIZE WRITE_SIZE; do
    echo "[counters] $tag $c"
    timeout -s KILL 200 rocprofv3 --pmc $c --output-format csv -d "$D/$c" -o run -- \
      python3 "$R/bench.py" --steps 5 --warmup 2 --no-cpu-baseline --calib-copy-mib 1024 $args \
      > "$D/$c.json" 2> "$D/$c.err"
    rc=$?
    if [ $rc -ne 0 ]; then
      if [ $rc -eq 124 ] || [ $rc -eq 137 ] || ! grep -q metric "$D/$c.json"; then
        echo "[counters] $tag $c failed (rc $rc)"; tail -5 "$D/$c.err"; exit $rc
      fi
      echo "[counters] $tag $c: profiler rc $rc after a complete run"
    fi
  done
done
echo "[counters] done"
