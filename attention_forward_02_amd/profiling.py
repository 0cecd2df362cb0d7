"""rocprofv3 summaries of the attention kernel, and the HBM traffic figure
the benchmark reports.

    bash attention_forward_02_amd/profile_run.sh WORKLOAD OUTDIR    (on a GPU)
    python -m attention_forward_02_amd.profiling OUTDIR WORKLOAD

The first command runs, on one MI355X, a kernel trace of the benchmark
command (`bench.py --no-cpu --no-configs --workload WORKLOAD`), five counter
passes of a short benchmark run (the fifth the L2 hits and misses), and the FETCH_SIZE / WRITE_SIZE passes of a plain
1 GiB device copy.  The second turns the CSV output into
`profiles/<kernel>_<WORKLOAD>.md` (the kernel the workload runs) and
records the calibrated HBM
bytes per launch in `profiles/traffic.json`, keyed by workload and stamped
with the digest of the kernel sources, so `bench.py` reports them only
while the kernel is the one that was profiled.

Counter conventions on MI355X (8 XCDs, 256 CUs, 1024 SIMDs):
* GRBM_GUI_ACTIVE is summed over the 8 XCDs: kernel cycles = value / 8.
* SQ_VALU_MFMA_BUSY_CYCLES is summed over all SIMDs, so the MFMA-busy
  fraction is value / (kernel cycles * 1024).
* FETCH_SIZE and WRITE_SIZE are KiB per dispatch.  They are scaled by what
  the same counter reads for the copy of a known byte count (the copy reads
  and writes 1 GiB).
"""

import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_JSON = os.path.join(PROFILES, "traffic.json")

KERNEL_SOURCES = ["csrc/attn_fwd_kernel.h", "csrc/attn_fwd_wide.h", "csrc/attn_fwd_d64.hip",
                  "csrc/attn_fwd_d128.hip", "csrc/attn_fwd_d128_wide.hip", "csrc/attn_fwd_d128_bc.hip", "csrc/attn_fwd_d256.hip",
                  "csrc/attn_fwd_d64_fp8.hip", "csrc/attn_fwd_d128_fp8.hip", "csrc/attn_fwd_d256_fp8.hip",
                  "csrc/attn_quant.hip", "csrc/attn_internal.h", "csrc/attn_fwd_splitkv.h",
                  "csrc/attn_fwd_splitkv.hip", "build.py"]
KERNEL = "attn::kernels::attn_fwd"  # every kernel of the library
N_XCD = 8
N_SIMD = 1024
COPY_BYTES = 1 << 30
HBM_PEAK = 8.0e12  # MI355X HBM3E, bytes/s

PMC_PASSES = [
    ["FETCH_SIZE"],
    ["WRITE_SIZE"],
    ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE"],
    ["SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"],
    ["TCC_HIT_sum", "TCC_MISS_sum"],
]


def _code_only(rel, text):
    """Source text without comments and with whitespace collapsed, so that
    editing a comment does not count as changing the kernel."""
    if rel.endswith(".py"):
        text = "\n".join(line.split("#", 1)[0] for line in text.splitlines())
    else:
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_digest():
    """sha256 over the code (comments and whitespace aside) of the kernel's
    source files and build options."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(PKG, rel)) as f:
            h.update(rel.encode() + b"\0" + _code_only(rel, f.read()).encode() + b"\0")
    return h.hexdigest()


def measured_traffic(workload):
    """Calibrated HBM bytes per launch for `workload`, or None when no
    profile exists or the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_JSON) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_digest") != kernel_digest():
        return None
    return rec


def _counters(path, name_filter):
    """Per-dispatch mean of every counter for kernels whose name contains
    `name_filter`."""
    agg = defaultdict(float)
    disp = set()
    with open(path) as f:
        for r in csv.DictReader(f):
            if name_filter in r["Kernel_Name"]:
                agg[r["Counter_Name"]] += float(r["Counter_Value"])
                disp.add(r["Dispatch_Id"])
    return {k: v / len(disp) for k, v in agg.items()}, len(disp)


def _one(pattern):
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def summarize(outdir, workload):
    from . import inputs
    w = inputs.WORKLOADS[workload]
    stats_rows = []
    with open(_one(os.path.join(outdir, "trace", "**", "*kernel_stats.csv"))) as f:
        for r in csv.DictReader(f):
            stats_rows.append(r)
    kern = [r for r in stats_rows if KERNEL in r["Name"]]
    if len(kern) != 1:
        raise RuntimeError(f"expected one {KERNEL} row in the kernel stats, found {len(kern)}")
    k = kern[0]
    kname = k["Name"].split("attn::kernels::")[1].split("<")[0]
    avg_ns = float(k["AverageNs"])
    c = {}
    ndisp = {}
    for i, names in enumerate(PMC_PASSES, 1):
        v, n = _counters(_one(os.path.join(outdir, f"pmc{i}", "**", "*counter_collection.csv")), KERNEL)
        c.update(v)
        ndisp[i] = n
    copy = {}
    for name in ("FETCH_SIZE", "WRITE_SIZE"):
        v, _ = _counters(_one(os.path.join(outdir, f"copy_{name}", "**", "*counter_collection.csv")), "copyBuffer")
        copy[name] = v[name]
    f_fetch = COPY_BYTES / (copy["FETCH_SIZE"] * 1024.0)
    f_write = COPY_BYTES / (copy["WRITE_SIZE"] * 1024.0)
    fetch_b = c["FETCH_SIZE"] * 1024.0 * f_fetch
    write_b = c["WRITE_SIZE"] * 1024.0 * f_write
    cycles = c["GRBM_GUI_ACTIVE"] / N_XCD
    mfma_busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * N_SIMD)
    lds_conf = c["SQ_LDS_BANK_CONFLICT"] / max(1.0, c["SQ_LDS_IDX_ACTIVE"])
    fl = inputs.flops(w["B"], w["H"], w["Nq"], w["Nk"], w["d"], w["causal"])
    elt = 1 if w["dtype"] == "e4m3" or w.get("smoothed") else 2
    alg_read = 3 * w["B"] * w["H"] * w["Nq"] * w["d"] * elt if w["Nq"] == w["Nk"] else None
    alg_write = w["B"] * w["H"] * w["Nq"] * (w["d"] * 2 + 4)
    tflops = fl / (avg_ns * 1e-9) / 1e12
    cmd_trace = (f"rocprofv3 --kernel-trace --stats --output-format csv -d {outdir}/trace -o run -- "
                 f"python3 bench.py --no-cpu --no-configs --workload {workload}")
    lines = [
        f"# {kname} on {workload}",
        "",
        f"Workload: B={w['B']} H={w['H']} Nq={w['Nq']} Nk={w['Nk']} d={w['d']} "
        f"causal={w['causal']} dtype={w['dtype']}; one launch = {fl:.4g} FLOP.",
        f"Kernel sources digest: `{kernel_digest()}` (code only: comments and whitespace aside)",
        "",
        "Made by (from the repository root, on one MI355X):",
        "",
        "```",
        f"bash attention_forward_02_amd/profile_run.sh {workload} {outdir}",
        f"python -m attention_forward_02_amd.profiling {outdir} {workload}",
        "```",
        "",
        "## Kernel trace (`--kernel-trace --stats`)",
        "",
        "```",
        cmd_trace,
        "```",
        "",
        "| kernel | calls | average ns | min ns | max ns | TFLOP/s at average |",
        "|---|---|---|---|---|---|",
        f"| `{k['Name']}` | {k['Calls']} | {avg_ns:.0f} | {float(k['MinNs']):.0f} | {float(k['MaxNs']):.0f} "
        f"| {tflops:.1f} |",
        "",
    ]
    others = [r for r in stats_rows if KERNEL not in r["Name"] and "attn::" in r["Name"]]
    if others:
        lines += ["Other kernels of the same step:", "",
                  "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
        for r in others:
            lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {float(r['MinNs']):.0f} "
                         f"| {float(r['MaxNs']):.0f} |")
        lines.append("")
    lines += [
        "## Counters (`--pmc`, one pass each, per dispatch)",
        "",
        "```",
    ]
    for i, names in enumerate(PMC_PASSES, 1):
        lines.append(f"timeout -s KILL 60 rocprofv3 --pmc {' '.join(names)} --output-format csv -d {outdir}/pmc{i} "
                     f"-o run -- python3 bench.py --steps 2 --warmup 1 --settle 0 --no-cpu --no-configs --workload {workload}")
    for name in ("FETCH_SIZE", "WRITE_SIZE"):
        lines.append(f"timeout -s KILL 60 rocprofv3 --pmc {name} --output-format csv -d {outdir}/copy_{name} "
                     f"-o run -- python3 bench.py --copy-mib 1024 --steps 2 --warmup 1")
    lines += [
        "```",
        "",
        "| counter | value per dispatch |",
        "|---|---|",
    ]
    for name in sorted(c):
        lines.append(f"| {name} | {c[name]:.6g} |")
    lines += [
        "",
        "| derived | value |",
        "|---|---|",
        f"| kernel cycles (GRBM_GUI_ACTIVE / 8 XCDs) | {cycles:.6g} |",
        f"| MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs)) | {100 * mfma_busy:.1f} % |",
        f"| LDS bank conflict cycles / LDS active cycles | {lds_conf:.4f} |",
        f"| VALU instructions per MFMA | {c['SQ_INSTS_VALU'] / max(1.0, c['SQ_INSTS_MFMA']):.2f} |",
        f"| L2 hit rate (TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)) | "
        f"{100 * c['TCC_HIT_sum'] / max(1.0, c['TCC_HIT_sum'] + c['TCC_MISS_sum']):.1f} % |",
        f"| copy calibration FETCH_SIZE (1 GiB read) | {copy['FETCH_SIZE']:.6g} KiB -> factor {f_fetch:.4f} |",
        f"| copy calibration WRITE_SIZE (1 GiB written) | {copy['WRITE_SIZE']:.6g} KiB -> factor {f_write:.4f} |",
        f"| HBM read per launch (calibrated) | {fetch_b / 1e6:.1f} MB |",
        f"| HBM write per launch (calibrated) | {write_b / 1e6:.1f} MB |",
        f"| HBM bandwidth (read + write per launch / average kernel time) | "
        f"{(fetch_b + write_b) / (avg_ns * 1e-9) / 1e9:.0f} GB/s, "
        f"{100 * (fetch_b + write_b) / (avg_ns * 1e-9) / HBM_PEAK:.1f} % of 8 TB/s |",
    ]
    if alg_read is not None:
        lines.append(f"| algorithmic read (Q, K, V once) / write (O, LSE) | {alg_read / 1e6:.1f} MB / "
                     f"{alg_write / 1e6:.1f} MB |")
    lines.append("")
    os.makedirs(PROFILES, exist_ok=True)
    md = os.path.join(PROFILES, f"{kname}_{workload}.md")
    # an earlier summary of the same workload under another kernel name (not
    # the tuning tables, profiles/tuning_<workload>.md)
    for old in glob.glob(os.path.join(PROFILES, f"attn_*_{workload}.md")):
        if old != md:
            os.remove(old)
    with open(md, "w") as f:
        f.write("\n".join(lines))
    try:
        with open(TRAFFIC_JSON) as f:
            traffic = json.load(f)
    except (OSError, ValueError):
        traffic = {}
    traffic[workload] = {
        "bytes": round(fetch_b + write_b),
        "fetch_bytes": round(fetch_b),
        "write_bytes": round(write_b),
        "fetch_factor": f_fetch,
        "write_factor": f_write,
        "kernel_digest": kernel_digest(),
        "kernel": kname,
        "summary": os.path.relpath(md, ROOT),
    }
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(traffic, f, indent=1, sort_keys=True)
        f.write("\n")
    print(f"wrote {md}; traffic {(fetch_b + write_b) / 1e6:.1f} MB per launch; "
          f"kernel avg {avg_ns / 1e3:.1f} us; MFMA busy {100 * mfma_busy:.1f} %")


# Counter passes of profile_variants.sh: wave states, then issue counts.
VARIANT_PASSES = [
    ["SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
     "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS", "GRBM_GUI_ACTIVE"],
    ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_LDS_LOAD_BANDWIDTH",
     "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE"],
]


def _per_kernel(path):
    """Per-dispatch mean of every counter, per attention kernel
    instantiation (the name up to its template arguments)."""
    agg = defaultdict(lambda: defaultdict(float))
    disp = defaultdict(set)
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if KERNEL not in name:
                continue
            key = name.split("attn::kernels::")[1].split("(")[0]
            agg[key][r["Counter_Name"]] += float(r["Counter_Value"])
            disp[key].add(r["Dispatch_Id"])
    return {k: {c: v / len(disp[k]) for c, v in d.items()} for k, d in agg.items()}


def summarize_variants(outdir, workload):
    """profiles/variants_<workload>.md: the counters of every kernel variant
    on one workload, from profile_variants.sh's passes over the tuner."""
    stats = {}
    with open(_one(os.path.join(outdir, "trace", "**", "*kernel_stats.csv"))) as f:
        for r in csv.DictReader(f):
            if KERNEL in r["Name"]:
                stats[r["Name"].split("attn::kernels::")[1].split("(")[0]] = float(r["AverageNs"])
    c = defaultdict(dict)
    for i in range(1, len(VARIANT_PASSES) + 1):
        for k, v in _per_kernel(_one(os.path.join(outdir, f"pmc{i}", "**", "*counter_collection.csv"))).items():
            c[k].update(v)
    tune = f"python3 -m attention_forward_02_amd.tune --workload {workload} --reps 3 --rounds 1"
    lines = [
        f"# Counters of every kernel variant on {workload}",
        "",
        f"Kernel sources digest: `{kernel_digest()}` (code only: comments and whitespace aside)",
        "",
        "Made by (from the repository root, on one MI355X):",
        "",
        "```",
        f"bash attention_forward_02_amd/profile_variants.sh {workload} {outdir}",
        f"python -m attention_forward_02_amd.profiling --variants {outdir} {workload}",
        "```",
        "",
        "which runs, each under its own time limit:",
        "",
        "```",
        f"rocprofv3 --kernel-trace --stats --output-format csv -d {outdir}/trace -o run -- {tune}",
    ]
    for i, names in enumerate(VARIANT_PASSES, 1):
        lines.append(f"rocprofv3 --pmc {' '.join(names)} --output-format csv -d {outdir}/pmc{i} -o run -- {tune}")
    lines += [
        "```",
        "",
        "Per dispatch, averaged over the tuner's launches of each kernel.  Wave-state",
        "fractions are of SQ_WAVE_CYCLES (every resident wave, a producer wave",
        "included): waiting = SQ_WAIT_ANY (on a waitcnt or a barrier), ready =",
        "SQ_WAIT_INST_ANY (an instruction ready but not issued), issuing =",
        "SQ_ACTIVE_INST_ANY.  LDS bytes from SQ_INSTS_LDS_LOAD_BANDWIDTH (64-byte",
        "units) over the kernel cycles and 256 CUs.",
        "",
        "| kernel | avg us (trace) | MFMA busy | waiting | ready | issuing | VALU instr / MFMA | LDS instr / MFMA "
        "| LDS read B/clk per CU | bank conflicts |",
        "|---|---|---|---|---|---|---|---|---|---|",
    ]
    for k in sorted(c, key=lambda k: stats.get(k, 1e30)):
        x = c[k]
        cyc = x["GRBM_GUI_ACTIVE"] / N_XCD
        wc = x["SQ_WAVE_CYCLES"]
        mf = max(1.0, x["SQ_INSTS_MFMA"])
        avg = f"{stats[k] / 1e3:.1f}" if k in stats else "-"
        lines.append(
            f"| `{k}` | {avg} | {100 * x['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * N_SIMD):.1f}% "
            f"| {100 * x['SQ_WAIT_ANY'] / wc:.1f}% | {100 * x['SQ_WAIT_INST_ANY'] / wc:.1f}% "
            f"| {100 * x['SQ_ACTIVE_INST_ANY'] / wc:.1f}% | {x['SQ_INSTS_VALU'] / mf:.2f} | {x['SQ_INSTS_LDS'] / mf:.2f} "
            f"| {x['SQ_INSTS_LDS_LOAD_BANDWIDTH'] * 64 / 256 / cyc:.1f} | {x['SQ_LDS_BANK_CONFLICT']:.0f} |")
    lines.append("")
    md = os.path.join(PROFILES, f"variants_{workload}.md")
    with open(md, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {md}")


if __name__ == "__main__":
    if len(sys.argv) == 4 and sys.argv[1] == "--variants":
        summarize_variants(sys.argv[2], sys.argv[3])
    elif len(sys.argv) == 3:
        summarize(sys.argv[1], sys.argv[2])
    else:
        sys.exit(__doc__)
