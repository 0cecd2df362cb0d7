"""Kernel-variant tuning: time every kernel variant the library builds for one
attention shape on the GPU and list them fastest first.

    python -m attention_forward_02_amd.tune --workload hd128_seq8k_f16 [--reps 20] [--write]
    python -m attention_forward_02_amd.tune --shape 2,16,8192,8192,64,bf16,causal

(--shape B,H,Nq,Nk,d,dtype[,causal]: seeded N(0, 1) inputs of that shape,
the way the named workloads are drawn, for a shape of one's own.)

The variants (ATTN_VARIANT_* in include/attn.h) compute the same forward pass
with different schedules: the pipelined kernel with a two- or four-stage K/V
ring, the sequential kernel, the split-key kernel, the pingpong kernel and
the producer-wave kernel.  The pages choose
tiles and stage counts by profiling ("Warp specialization" concept card, its
notes on tile sizes and on the three-stage variants); this does the same on
the device at hand.  The library's default (ATTN_VARIANT_AUTO) encodes the
choices measured so far; the tuner shows whether a shape would gain from
another one, which a caller can then request with ``attention(...,
variant=...)``.

Before it is timed, every variant's output is compared with the default
variant's on the same inputs (the two may differ only by rounding order):
fp16/bf16 max |dO| <= 8e-3 plus one output ulp and max |dLSE| <= 2e-3, E4M3
relative RMSE <= 3e-2.  A variant that disagrees is reported, not timed.

Timing: the GPU first runs the default variant for about half a second
(clocks settle; a cold start reads up to 15% slow), then every variant is
timed in ``rounds`` interleaved rounds of ``reps`` launches (HIP events on
the current stream); the table gives each variant's best round.  With
--write the table goes to profiles/tuning_<workload>.md.
"""

import argparse
import math
import os
import sys

from . import binding as b

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
VARIANTS = [b.ATTN_VARIANT_AUTO, b.ATTN_VARIANT_PIPELINED, b.ATTN_VARIANT_PIPELINED_4STAGE,
            b.ATTN_VARIANT_SEQUENTIAL, b.ATTN_VARIANT_SPLIT, b.ATTN_VARIANT_PINGPONG,
            b.ATTN_VARIANT_PRODUCER, b.ATTN_VARIANT_WIDE, b.ATTN_VARIANT_SEQUENTIAL_BC32,
            b.ATTN_VARIANT_SEQUENTIAL_BC128, b.ATTN_VARIANT_PIPELINED_3STAGE]


def _agree(o, lse, o_ref, lse_ref, fp8):
    import torch
    dl = (lse - lse_ref).abs()
    finite = torch.isfinite(lse_ref)
    if not torch.equal(torch.isfinite(lse), finite):
        return False, "LSE finiteness differs"
    dlm = float(dl[finite].max()) if bool(finite.any()) else 0.0
    of, rf = o.float(), o_ref.float()
    if fp8:
        rel = float((of - rf).norm() / rf.norm().clamp_min(1e-30))
        return rel <= 3e-2 and dlm <= 2e-3, f"rel RMSE {rel:.3g}, max |dLSE| {dlm:.3g}"
    ulp = torch.finfo(o.dtype).eps * rf.abs().clamp_min(1.0)
    bad = ((of - rf).abs() > 8e-3 + ulp).sum().item()
    return bad == 0 and dlm <= 2e-3, f"max |dO| {float((of - rf).abs().max()):.3g}, max |dLSE| {dlm:.3g}"


def _time(fn, reps, st):
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def tune(q, k, v, causal=False, scale=None, descale=None, reps=20, rounds=3, settle_s=0.5, stream=None):
    """Time every variant built for these device tensors (as for
    ``attention``).  Returns a list of dicts (variant, name, ms, tflops,
    check), the default first, then the others fastest first."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    code = b._dtype_code(q)
    fp8 = code == b.ATTN_FP8_E4M3
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    flops = 4.0 * B * H * Nq * Nk * d / (2.0 if causal else 1.0)
    st = torch.cuda.current_stream() if stream is None else stream
    ref = None
    rows = []
    for var in VARIANTS:
        if not b.attn_variant_available(d, code, var):
            continue
        o, lse = b.attention(q, k, v, causal, scale, descale, st, variant=var)
        torch.cuda.synchronize()
        if ref is None:
            ref = (o, lse)
            ok, msg = True, "reference"
        else:
            ok, msg = _agree(o, lse, ref[0], ref[1], fp8)
        row = {"variant": var, "name": b.VARIANT_NAMES[var], "ms": None, "tflops": None, "check": msg}
        if not ok:
            row["check"] = "DISAGREES: " + msg
        rows.append(row)
    call = lambda var: (lambda: b.attention(q, k, v, causal, scale, descale, st, variant=var))
    # settle: run the default until about settle_s seconds have passed
    spent, n = 0.0, 1
    while spent < settle_s * 1e3:
        spent += _time(call(b.ATTN_VARIANT_AUTO), n, st) * n
        n = min(2 * n, 1024)
    for _ in range(rounds):
        for row in rows:
            if row["check"].startswith("DISAGREES"):
                continue
            ms = _time(call(row["variant"]), reps, st)
            if row["ms"] is None or ms < row["ms"]:
                row["ms"], row["tflops"] = ms, flops / (ms * 1e-3) / 1e12
    head, rest = rows[:1], rows[1:]
    rest.sort(key=lambda r: (r["ms"] is None, r["ms"] or 0.0))
    return head + rest


def _table(rows, workload, cmd):
    auto = rows[0]["ms"]
    lines = [f"# Kernel variants on {workload}", "", "Made by (from the repository root, on one MI355X):", "",
             "```", cmd, "```", "",
             "Best of the interleaved rounds, after the clocks settled.", "",
             "| variant | ms per launch | TFLOP/s | vs default | check against the default's output |",
             "|---|---|---|---|---|"]
    for r in rows:
        if r["ms"] is None:
            lines.append(f"| {r['name']} | — | — | — | {r['check']} |")
        else:
            lines.append(f"| {r['name']} | {r['ms']:.4f} | {r['tflops']:.1f} | {auto / r['ms']:.3f}x | {r['check']} |")
    lines.append("")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", default="hd128_seq8k_f16")
    ap.add_argument("--shape", help="B,H,Nq,Nk,d,dtype[,causal] instead of a named workload")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--rounds", type=int, default=3)
    ap.add_argument("--write", action="store_true", help="write profiles/tuning_<workload>.md")
    args = ap.parse_args(argv)
    import numpy as np
    import torch
    from . import inputs
    if args.shape:
        f = args.shape.split(",")
        if len(f) not in (6, 7) or (len(f) == 7 and f[6] != "causal"):
            sys.exit("--shape takes B,H,Nq,Nk,d,dtype[,causal]")
        B, H, Nq, Nk, d = (int(x) for x in f[:5])
        inp = inputs.make(B, H, Nq, Nk, d, f[5], seed=1, causal=len(f) == 7)
        label = args.shape
    else:
        if inputs.WORKLOADS[args.workload].get("smoothed"):
            sys.exit("the block-scaled path has a single kernel variant")
        inp = inputs.make_workload(args.workload)
        label = args.workload
    dev = torch.device("cuda:0")
    if inp.dtype == "e4m3":
        up = lambda x: torch.from_numpy(x).view(torch.float8_e4m3fn).to(dev)
        desc = tuple(float(x) for x in inp.descale)
    else:
        dt = torch.float16 if inp.dtype == "f16" else torch.bfloat16
        up = lambda x: torch.from_numpy(x.view(np.int16)).view(dt).to(dev)
        desc = None
    rows = tune(up(inp.q), up(inp.k), up(inp.v), inp.causal, float(inp.scale), desc, reps=args.reps,
                rounds=args.rounds)
    which = f"--shape {args.shape}" if args.shape else f"--workload {args.workload}"
    cmd = f"python -m attention_forward_02_amd.tune {which} --reps {args.reps} --rounds {args.rounds} --write"
    text = _table(rows, label, cmd)
    print(text, flush=True)
    if args.write:
        name = args.workload if not args.shape else "shape_" + args.shape.replace(",", "_")
        with open(os.path.join(ROOT, "profiles", f"tuning_{name}.md"), "w") as f:
            f.write(text)


if __name__ == "__main__":
    main()
