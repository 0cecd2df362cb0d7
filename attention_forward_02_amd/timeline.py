"""Timeline probe: where a workgroup's cycles go, step by step.

    python -m attention_forward_02_amd.timeline --workload causal_d64_bf16 [--write]
    python -m attention_forward_02_amd.timeline --workload hd128_seq8k_f16 [--write]

``libattn_timeline.so`` (built by build.py from csrc/attn_timeline.hip) holds
two of the library's kernels compiled with their shader-clock trace points
(``Timeline`` in attn_fwd_kernel.h; the attention library's own build has
none): the sequential 128-key kernel at d = 64, bfloat16, causal (the
default of causal_d64_bf16) and the producer-wave kernel at d = 128,
binary16 (the default of hd128_seq8k_f16).  Lane 0 of every wave records
the shader clock at kernel entry, after its set-up, after every step and
after the output is stored, plus the cycles it spent waiting at the step
barriers.

The probe first checks that the traced kernel's outputs equal those of the
same library variant, requested explicitly, bit for bit (the trace points
change timing, not arithmetic), and reports both kernels' times, so the
trace overhead is visible.  Then, after about a
second of launches (the clocks settle), it records one launch and writes:

* causal_d64_bf16: per query tile length (steps per workgroup), the median
  cycles of the set-up, of each step and of the epilogue, over the waves of
  every workgroup with that many steps;
* hd128_seq8k_f16: per wave of the workgroup (eight consumers, one
  producer), the median cycles per step and the share of them spent waiting
  at the step barrier.

With --write the table goes to profiles/timeline_<workload>.md.
"""

import argparse
import ctypes
import os
import sys
import time

import numpy as np

from . import binding as b
from . import inputs

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libattn_timeline.so")

# workload -> (C entry point, head dim, dtype, causal, waves and query rows
# per workgroup, the library variant the traced kernel is)
PROBES = {
    "causal_d64_bf16": ("attn_timeline_seq_d64_bf16_causal", 64, "bf16", True, 4, 128,
                        b.ATTN_VARIANT_SEQUENTIAL_BC128),
    "hd128_seq8k_f16": ("attn_timeline_producer_d128_f16", 128, "f16", False, 9, 256, b.ATTN_VARIANT_PRODUCER),
}

_lib = None


def load_library(path=LIB):
    """The timeline library; raises when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built: run python -m attention_forward_02_amd.build")
        lib = ctypes.CDLL(path)
        vp, ci, ull = ctypes.c_void_p, ctypes.c_int, ctypes.c_ulonglong
        for name, *_ in PROBES.values():
            fn = getattr(lib, name)
            fn.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ctypes.c_float, vp, ull, vp]
            fn.restype = ci
        lib.attn_timeline_slots.restype = ci
        _lib = lib
    return _lib


def run(workload, q, k, v, scale, timeline, stream=None):
    """One launch of the traced kernel for ``workload`` on device tensors
    q, k, v ([B, H, N, d]); returns (o, lse).  ``timeline`` is an int64
    device tensor of at least workgroups x waves x slots entries."""
    import torch
    name, d, dtype, causal, waves, rows, _ = PROBES[workload]
    b._check_qkv(q, k, v)
    B, H, Nq, dq = q.shape
    if dq != d or q.dtype != (torch.bfloat16 if dtype == "bf16" else torch.float16):
        raise ValueError(f"the {workload} probe takes d = {d} {dtype} inputs")
    if not (timeline.is_cuda and timeline.dtype == torch.int64 and timeline.is_contiguous()
            and timeline.device == q.device):
        raise ValueError("timeline must be a contiguous int64 tensor on q's device")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    st = torch.cuda.current_stream() if stream is None else stream
    status = getattr(load_library(), name)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                           B, H, Nq, k.shape[2], float(scale), timeline.data_ptr(),
                                           timeline.numel() * 8, st.cuda_stream)
    if status != b.ATTN_OK:
        raise b.AttnError(status)
    return o, lse


def _seq_table(t, slots):
    """Per steps-per-workgroup medians (sequential kernel)."""
    nt = t[:, 0, slots - 2]
    steps = slots - 6
    lines = ["| steps per workgroup | workgroups | set-up | " + " | ".join(f"step {j}" for j in range(int(nt.max())))
             + " | epilogue | total | barrier wait |",
             "|---" * (int(nt.max()) + 6) + "|"]
    for n in sorted(set(nt.tolist())):
        g = t[nt == n]                                   # [workgroups, waves, slots]
        n = int(n)
        if n < 1 or n > steps:
            continue
        marks = g[:, :, 1:2 + n]                         # after set-up, after each step
        per = np.diff(marks, axis=2)
        cells = [f"{np.median(g[:, :, 1] - g[:, :, 0]):.0f}"]
        cells += [f"{np.median(per[:, :, j]):.0f}" for j in range(n)]
        cells += [""] * (int(nt.max()) - n)
        cells += [f"{np.median(g[:, :, slots - 3] - g[:, :, 1 + n]):.0f}",
                  f"{np.median(g[:, :, slots - 3] - g[:, :, 0]):.0f}",
                  f"{np.median(g[:, :, slots - 4]):.0f}"]
        lines.append(f"| {n} | {g.shape[0]} | " + " | ".join(cells) + " |")
    return lines


def _producer_table(t, slots):
    """Per-wave medians (producer-wave kernel)."""
    nt = t[:, :, slots - 2].astype(np.float64)
    loop = (t[:, :, slots - 3] - t[:, :, 1]).astype(np.float64)
    wait = t[:, :, slots - 4].astype(np.float64)
    lines = ["| wave | role | cycles per step | barrier wait per step | barrier wait share |", "|---|---|---|---|---|"]
    for w in range(t.shape[1]):
        role = "consumer" if w < t.shape[1] - 1 else "producer"
        lines.append(f"| {w} | {role} | {np.median(loop[:, w] / nt[:, w]):.0f} | "
                     f"{np.median(wait[:, w] / nt[:, w]):.0f} | {np.median(wait[:, w] / loop[:, w]):.1%} |")
    return lines


def profile(workload, settle_s=1.0, reps=20):
    """Runs the probe on the named workload's inputs; returns (markdown
    lines, summary dict)."""
    import torch
    if workload not in PROBES:
        raise ValueError(f"no timeline probe for {workload}; choose from {sorted(PROBES)}")
    name, d, dtype, causal, waves, rows, variant = PROBES[workload]
    w = inputs.WORKLOADS[workload]
    inp = inputs.make_workload(workload)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    up = lambda x: torch.from_numpy(x.view(np.int16)).view(tdt).to(dev)
    q, k, v = up(inp.q), up(inp.k), up(inp.v)
    scale = float(inp.scale)
    slots = load_library().attn_timeline_slots()
    wgs = w["B"] * w["H"] * (-(-w["Nq"] // rows))
    tl = torch.zeros(wgs * waves * slots, dtype=torch.int64, device=dev)
    o_ref, lse_ref = b.attention(q, k, v, causal, scale, variant=variant)
    o, lse = run(workload, q, k, v, scale, tl)
    torch.cuda.synchronize()
    same = torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(lse, lse_ref)
    if not same:
        raise RuntimeError("the traced kernel's output differs from the library's")
    st = torch.cuda.current_stream()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    t0 = time.time()
    while time.time() - t0 < settle_s:
        run(workload, q, k, v, scale, tl)
        torch.cuda.synchronize()
    ms_probe = timed(lambda: run(workload, q, k, v, scale, tl))
    ms_lib = timed(lambda: b.attention(q, k, v, causal, scale, variant=variant))
    tl.zero_()
    run(workload, q, k, v, scale, tl)
    torch.cuda.synchronize()
    t = tl.cpu().numpy().reshape(wgs, waves, slots)
    table = _seq_table(t, slots) if waves == 4 else _producer_table(t, slots)
    head = [f"# Timeline of the {workload} default kernel",
            "",
            f"Workload: B={w['B']} H={w['H']} Nq={w['Nq']} Nk={w['Nk']} d={w['d']} causal={w['causal']} "
            f"dtype={w['dtype']}; {wgs} workgroups of {waves} waves.",
            "",
            "Made by (from the repository root, on one MI355X):",
            "",
            "```",
            f"python -m attention_forward_02_amd.timeline --workload {workload} --write",
            "```",
            "",
            f"The traced kernel's outputs equal the library's bit for bit. Launch times (events, {reps} launches, "
            f"after {settle_s:.0f} s of launches): traced {ms_probe:.4f} ms, library {ms_lib:.4f} ms. One recorded "
            "launch; shader-clock cycles, medians over the waves of the workgroups in each row. A step is "
            "counted from the end of the previous one (or of the set-up) to the end of its last instruction "
            "issue, so the MFMAs it leaves in flight fall into the next part; the barrier wait is the time "
            "between reaching a step's barrier and passing it, summed over the steps.",
            ""]
    return head + table + [""], {"ms_probe": ms_probe, "ms_library": ms_lib}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", default="causal_d64_bf16", choices=sorted(PROBES))
    ap.add_argument("--write", action="store_true", help="write profiles/timeline_<workload>.md")
    args = ap.parse_args(argv)
    lines, _ = profile(args.workload)
    text = "\n".join(lines)
    print(text, flush=True)
    if args.write:
        with open(os.path.join(ROOT, "profiles", f"timeline_{args.workload}.md"), "w") as f:
            f.write(text)


if __name__ == "__main__":
    sys.exit(main())
