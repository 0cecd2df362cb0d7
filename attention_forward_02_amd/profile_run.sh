#!/bin/bash
# rocprofv3 passes behind profiles/<kernel>_<WORKLOAD>.md (one MI355X).
#   bash attention_forward_02_amd/profile_run.sh WORKLOAD OUTDIR
# Then: python -m attention_forward_02_amd.profiling OUTDIR WORKLOAD
# Each pass runs under its own time limit and the script stops at the first
# failing pass.  Counter passes hold one counter group each.
set -o pipefail
WL=${1:?workload}
OUT=${2:?output directory}
ROOT=$(cd "$(dirname "$0")/.." && pwd)
cd "$ROOT" || exit 1
mkdir -p "$OUT"
export TMPDIR=/tmp

echo "[profile] kernel trace: $WL"
timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv -d "$OUT/trace" -o run -- \
  python3 bench.py --no-cpu --no-configs --workload "$WL" > "$OUT/trace.log" 2>&1 || { tail -20 "$OUT/trace.log"; exit 1; }

i=0
for pmc in "FETCH_SIZE" "WRITE_SIZE" \
           "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS GRBM_GUI_ACTIVE" \
           "SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_BUSY_CYCLES GRBM_GUI_ACTIVE" \
           "TCC_HIT_sum TCC_MISS_sum"; do
  i=$((i + 1))
  echo "[profile] counter pass $i: $pmc"
  timeout -s KILL 60 rocprofv3 --pmc $pmc --output-format csv -d "$OUT/pmc$i" -o run -- \
    python3 bench.py --steps 2 --warmup 1 --settle 0 --no-cpu --no-configs --workload "$WL" > "$OUT/pmc$i.log" 2>&1 \
    || { tail -20 "$OUT/pmc$i.log"; exit 1; }
done

for pmc in FETCH_SIZE WRITE_SIZE; do
  echo "[profile] copy calibration: $pmc"
  timeout -s KILL 60 rocprofv3 --pmc $pmc --output-format csv -d "$OUT/copy_$pmc" -o run -- \
    python3 bench.py --copy-mib 1024 --steps 2 --warmup 1 > "$OUT/copy_$pmc.log" 2>&1 \
    || { tail -20 "$OUT/copy_$pmc.log"; exit 1; }
done
echo "[profile] done: $OUT"
