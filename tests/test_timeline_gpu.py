"""The timeline probe (libattn_timeline.so, attention_forward_02_amd/timeline.py)
on small ragged shapes: the traced kernels' outputs equal the library's bit
for bit, and every wave's trace is ordered (entry <= set-up <= each step <=
end) with the workgroup's step count."""

import numpy as np
import pytest
import torch

from attention_forward_02_amd import attention, inputs, timeline
from gpu_helpers import say, upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("workload,B,H,N", [("causal_d64_bf16", 1, 2, 300), ("hd128_seq8k_f16", 1, 2, 600)])
def test_timeline_probe_matches_library(workload, B, H, N):
    _, d, dtype, causal, waves, rows, variant = timeline.PROBES[workload]
    say(f"[gpu] timeline {workload}: B={B} H={H} N={N} d={d} {dtype} causal={causal}")
    inp = inputs.make(B, H, N, N, d, dtype, seed=31, causal=causal)
    q, k, v = (upload(t, dtype) for t in (inp.q, inp.k, inp.v))
    slots = timeline.load_library().attn_timeline_slots()
    wgs = B * H * (-(-N // rows))
    tl = torch.zeros(wgs * waves * slots, dtype=torch.int64, device="cuda")
    o, lse = timeline.run(workload, q, k, v, float(inp.scale), tl)
    o_ref, lse_ref = attention(q, k, v, causal=causal, scale=float(inp.scale), variant=variant)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(lse, lse_ref)
    t = tl.cpu().numpy().reshape(wgs, waves, slots)
    bn = 128 if workload == "causal_d64_bf16" else 64
    for wg in range(wgs):
        qt = wg % (-(-N // rows))
        for w in range(waves):
            nt = int(t[wg, w, slots - 2])
            assert nt >= 1 and nt <= -(-N // bn)
            marks = [t[wg, w, 0], t[wg, w, 1]]
            if w < waves - 1 or workload == "causal_d64_bf16":   # consumers mark every step
                marks += [t[wg, w, 2 + j] for j in range(min(nt, slots - 6))]
            marks.append(t[wg, w, slots - 3])
            assert all(a <= b for a, b in zip(marks, marks[1:])), (wg, w, marks)
            assert t[wg, w, slots - 4] >= 0
    say(f"[gpu] timeline {workload}: {wgs} workgroups traced, outputs bitwise equal to the library's")


def test_timeline_rejects_bad_arguments():
    inp = inputs.make(1, 1, 64, 64, 64, "bf16", seed=1, causal=True)
    q, k, v = (upload(t, "bf16") for t in (inp.q, inp.k, inp.v))
    with pytest.raises(ValueError):
        timeline.run("causal_d64_bf16", q, k, v, 0.125, torch.zeros(8, dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError):
        timeline.run("hd128_seq8k_f16", q, k, v, 0.125, torch.zeros(10 ** 4, dtype=torch.int64, device="cuda"))
    # too small a trace buffer: rejected by the library before launching
    with pytest.raises(RuntimeError):
        timeline.run("causal_d64_bf16", q, k, v, 0.125, torch.zeros(8, dtype=torch.int64, device="cuda"))
