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
