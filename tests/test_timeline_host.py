"""The timeline probe's library on the CPU: it loads, and rejects invalid
arguments with the library's status codes before touching the device (the
fake device addresses below are never dereferenced)."""

import os

import pytest

from attention_forward_02_amd import binding as b
from attention_forward_02_amd import timeline

Q, K, V, O, L, T = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000, 0x60000000


def _lib():
    if not os.path.exists(timeline.LIB):
        pytest.fail("libattn_timeline.so is not built (python -m attention_forward_02_amd.build)")
    return timeline.load_library()


def test_timeline_library_rejects_before_launch():
    lib = _lib()
    assert lib.attn_timeline_slots() == 64
    for name, _, _, _, waves, rows, _ in timeline.PROBES.values():
        f = getattr(lib, name)
        # one workgroup of `rows` query rows needs waves x 64 counters of 8 bytes
        need = waves * 64 * 8
        assert f(None, K, V, O, L, 1, 1, rows, 128, 0.1, T, need, None) == b.ATTN_ERR_NULL
        assert f(Q, K, V, O, L, 1, 1, rows, 128, 0.1, None, need, None) == b.ATTN_ERR_NULL
        assert f(Q, K, V, O, L, 0, 1, rows, 128, 0.1, T, need, None) == b.ATTN_ERR_SHAPE
        assert f(Q, K, V, O, L, 1, 1, rows, 0, 0.1, T, need, None) == b.ATTN_ERR_SHAPE
        assert f(Q, K, V, O, L, 1, 1, rows, 128, 0.1, T, need - 8, None) == b.ATTN_ERR_SHAPE
        assert f(Q, K, V, O, L, 1, 1, rows + 1, 128, 0.1, T, need, None) == b.ATTN_ERR_SHAPE
        assert f(Q, K, V, O, L, 1 << 16, 1 << 12, 1 << 10, 128, 0.1, T, 1 << 62, None) == b.ATTN_ERR_SHAPE


def test_timeline_cli_names_its_workloads():
    assert set(timeline.PROBES) <= set(__import__("attention_forward_02_amd.inputs", fromlist=["x"]).WORKLOADS)
    with pytest.raises(SystemExit):
        timeline.main(["--workload", "tiny_d64_f16"])
