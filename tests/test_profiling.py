"""The benchmark's HBM traffic figure comes from committed counter passes
and is withheld once the kernel sources no longer match them."""

import json

from attention_forward_02_amd import profiling


def test_traffic_follows_kernel_digest(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(profiling, "TRAFFIC_JSON", str(path))
    assert profiling.measured_traffic("hd128_seq8k_f16") is None          # no file
    rec = {"bytes": 123, "kernel_digest": profiling.kernel_digest()}
    path.write_text(json.dumps({"hd128_seq8k_f16": rec, "other": dict(rec, kernel_digest="0" * 64)}))
    assert profiling.measured_traffic("hd128_seq8k_f16")["bytes"] == 123  # current kernel
    assert profiling.measured_traffic("other") is None                    # stale kernel
    assert profiling.measured_traffic("missing") is None


def test_digest_covers_kernel_sources():
    assert len(profiling.kernel_digest()) == 64
    assert "csrc/attn_fwd_kernel.h" in profiling.KERNEL_SOURCES


def test_digest_ignores_comments_not_code():
    src = "int f(int x) {  // doubles\n  return 2 * x; /* a note */\n}\n"
    assert profiling._code_only("k.h", src) == profiling._code_only("k.h", src.replace("doubles", "twice"))
    assert profiling._code_only("k.h", src) != profiling._code_only("k.h", src.replace("2 * x", "3 * x"))
    py = "FLAGS = ['-O3']  # optimise\n"
    assert profiling._code_only("build.py", py) == profiling._code_only("build.py", py.replace("optimise", "fast"))
    assert profiling._code_only("build.py", py) != profiling._code_only("build.py", py.replace("-O3", "-O2"))


def test_variant_summary_from_counter_files(tmp_path, monkeypatch):
    """profiles/variants_<workload>.md: one row per kernel instantiation,
    ratios taken per dispatch from the two counter passes."""
    import csv

    monkeypatch.setattr(profiling, "PROFILES", str(tmp_path / "profiles"))
    (tmp_path / "profiles").mkdir()
    out = tmp_path / "run"
    k1 = "void attn::kernels::attn_fwd_a<128, 0, false>(attn::kernels::Params)"
    k2 = "void attn::kernels::attn_fwd_b<128, 0, false>(attn::kernels::Params)"
    (out / "trace").mkdir(parents=True)
    with open(out / "trace" / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, ["Name", "Calls", "AverageNs"])
        w.writeheader()
        w.writerow({"Name": k1, "Calls": 2, "AverageNs": 2000.0})
        w.writerow({"Name": k2, "Calls": 1, "AverageNs": 1000.0})
    cyc = 1000.0
    vals = {k1: dict(SQ_WAVE_CYCLES=100, SQ_WAIT_ANY=50, SQ_WAIT_INST_ANY=20, SQ_ACTIVE_INST_ANY=30,
                     SQ_ACTIVE_INST_VALU=10, SQ_ACTIVE_INST_LDS=5, SQ_WAIT_INST_LDS=1, GRBM_GUI_ACTIVE=8 * cyc,
                     SQ_VALU_MFMA_BUSY_CYCLES=0.5 * cyc * 1024, SQ_INSTS_VALU=40, SQ_INSTS_MFMA=10, SQ_INSTS_LDS=15,
                     SQ_INSTS_LDS_LOAD_BANDWIDTH=4000, SQ_LDS_BANK_CONFLICT=0, SQ_LDS_IDX_ACTIVE=1),
            k2: dict(SQ_WAVE_CYCLES=100, SQ_WAIT_ANY=10, SQ_WAIT_INST_ANY=10, SQ_ACTIVE_INST_ANY=80,
                     SQ_ACTIVE_INST_VALU=10, SQ_ACTIVE_INST_LDS=5, SQ_WAIT_INST_LDS=1, GRBM_GUI_ACTIVE=8 * cyc,
                     SQ_VALU_MFMA_BUSY_CYCLES=0.25 * cyc * 1024, SQ_INSTS_VALU=30, SQ_INSTS_MFMA=10, SQ_INSTS_LDS=5,
                     SQ_INSTS_LDS_LOAD_BANDWIDTH=2000, SQ_LDS_BANK_CONFLICT=0, SQ_LDS_IDX_ACTIVE=1)}
    for i, names in enumerate(profiling.VARIANT_PASSES, 1):
        (out / f"pmc{i}").mkdir()
        with open(out / f"pmc{i}" / "run_counter_collection.csv", "w", newline="") as f:
            w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for disp, k in ((1, k1), (2, k1), (3, k2)):  # two dispatches of k1: per-dispatch means
                for name in names:
                    w.writerow({"Dispatch_Id": disp, "Kernel_Name": k, "Counter_Name": name,
                                "Counter_Value": vals[k][name]})
    profiling.summarize_variants(str(out), "hd128_seq8k_f16")
    rows = [ln for ln in (tmp_path / "profiles" / "variants_hd128_seq8k_f16.md").read_text().splitlines()
            if ln.startswith("| `attn_fwd_")]
    # fastest first (trace averages), then MFMA busy, waiting, ready, issuing, VALU/MFMA, LDS/MFMA,
    # LDS bytes per clock per CU (64-byte units over 256 CUs), bank conflicts
    assert rows[0].startswith("| `attn_fwd_b<128, 0, false>` | 1.0 | 25.0% | 10.0% | 10.0% | 80.0% | 3.00 | 0.50 | 0.5 | 0 |")
    assert rows[1].startswith("| `attn_fwd_a<128, 0, false>` | 2.0 | 50.0% | 50.0% | 20.0% | 30.0% | 4.00 | 1.50 | 1.0 | 0 |")
