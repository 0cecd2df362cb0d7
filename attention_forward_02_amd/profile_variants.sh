#!/bin/bash
# rocprofv3 passes behind profiles/variants_<WORKLOAD>.md (one MI355X): the
# tuner launches every kernel variant built for the workload, and each pass
# records every launch.
#   bash attention_forward_02_amd/profile_variants.sh WORKLOAD OUTDIR
# Then: python -m attention_forward_02_amd.profiling --variants OUTDIR WORKLOAD
# Each pass runs under its own time limit and the script stops at the first
# failing pass.  The counter lists are VARIANT_PASSES in profiling.py.
set -o pipefail
WL=${1:?workload}
OUT=${2:?output directory}
ROOT=$(cd "$(dirname "$0")/.." && pwd)
cd "$ROOT" || exit 1
mkdir -p "$OUT"
export TMPDIR=/tmp
TUNE="python3 -m attention_forward_02_amd.tune --workload $WL --reps 3 --rounds 1"

echo "[profile] kernel trace: $WL (all variants)"
timeout -k 10 150 rocprofv3 --kernel-trace --stats --output-format csv -d "$OUT/trace" -o run -- \
  $TUNE > "$OUT/trace.log" 2>&1 || { tail -20 "$OUT/trace.log"; exit 1; }

i=0
for pmc in "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS GRBM_GUI_ACTIVE" \
           "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_LDS_LOAD_BANDWIDTH SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE"; do
  i=$((i + 1))
  echo "[profile] counter pass $i: $pmc"
  timeout -s KILL 150 rocprofv3 --pmc $pmc --output-format csv -d "$OUT/pmc$i" -o run -- \
    $TUNE > "$OUT/pmc$i.log" 2>&1 || { tail -20 "$OUT/pmc$i.log"; exit 1; }
done
echo "[profile] done: $OUT"
