"""The forward under HIP graph capture: launches of attn_fwd, of
attn_fwd_splitkv (split and merge kernels on a caller workspace) and of the
allocation-free attn_fwd_splitkv_noalloc are captured in a graph, which is
replayed three times with eager calls and synchronisations between the
replays; every replay must give the eager call's outputs bit for bit, and
those must meet the oracle's gates.  None of these calls records a memset
or an allocation, so the captured graph holds kernel launches only."""

import numpy as np
import pytest
import torch

from attention_forward_02_amd import inputs
from attention_forward_02_amd.binding import (ATTN_BF16, ATTN_F16, ATTN_OK, attn_fwd, attn_fwd_splitkv,
                                              attn_fwd_splitkv_noalloc, attn_fwd_splitkv_num_splits,
                                              attn_fwd_splitkv_workspace_bytes)
from gpu_helpers import compare, dequant, oracle_all_heads, say, upload

pytestmark = pytest.mark.gpu

CODES = {"f16": ATTN_F16, "bf16": ATTN_BF16}


def _replays_match(call, outs, label, launches=3):
    """Eager call, then a graph of `launches` calls replayed three times."""
    st = torch.cuda.current_stream()
    call(st)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream()
        for _ in range(launches):
            call(cap)
    for r in range(3):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for t, t_ref in zip(outs, ref):
            assert torch.equal(t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16),
                               t_ref.view(torch.int32) if t.dtype == torch.float32 else t_ref.view(torch.int16)), \
                f"{label}: graph replay {r} differs from the eager call"
        call(st)                     # eager work between the replays
        torch.cuda.synchronize()
    say(f"[gpu] {label}: three graph replays of {launches} launches equal the eager call")


def _check_oracle(inp, o, lse, label):
    qq, kk, vv = dequant(inp)
    o_ref, l_ref = oracle_all_heads(qq, kk, vv, inp.causal, float(inp.scale))
    stats = compare(o.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy(), o_ref, l_ref, inp.dtype,
                    label)
    say(f"[gpu] {label}: {stats}")


def _outputs(inp):
    dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float16
    return (torch.empty((inp.B, inp.H, inp.Nq, inp.d), dtype=dt, device="cuda"),
            torch.empty((inp.B, inp.H, inp.Nq), dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("d,dtype,causal,n", [(64, "f16", True, 300), (128, "bf16", False, 520), (256, "f16", True, 200)])
def test_attn_fwd_in_a_graph(d, dtype, causal, n):
    label = f"graph attn_fwd d={d} {dtype} causal={causal} N={n}"
    say(f"[gpu] {label}: B=1 H=2")
    inp = inputs.make(1, 2, n, n, d, dtype, seed=90 + d, causal=causal)
    q, k, v = (upload(t, dtype) for t in (inp.q, inp.k, inp.v))
    o, lse = _outputs(inp)

    def call(s):
        assert attn_fwd(q, k, v, o, lse, inp.B, inp.H, inp.Nq, inp.Nk, d, causal, float(inp.scale), CODES[dtype],
                        s) == ATTN_OK

    _replays_match(call, (o, lse), label)
    _check_oracle(inp, o, lse, label)


@pytest.mark.parametrize("noalloc", [False, True])
def test_splitkv_in_a_graph(noalloc):
    inp = inputs.make(1, 2, 64, 3000, 128, "f16", seed=95, causal=True)
    args = (inp.B, inp.H, inp.Nq, inp.Nk, inp.d, True, float(inp.scale), ATTN_F16, 1.0, 1.0, 1.0, 0)
    ns = attn_fwd_splitkv_num_splits(inp.B, inp.H, inp.Nq, inp.Nk, inp.d, True, ATTN_F16, 0)
    need = attn_fwd_splitkv_workspace_bytes(inp.B, inp.H, inp.Nq, inp.Nk, inp.d, True, ATTN_F16, 0)
    label = f"graph attn_fwd_splitkv{'_noalloc' if noalloc else ''} ({ns} splits)"
    say(f"[gpu] {label}: B=1 H=2 Nq=64 Nk=3000 d=128 f16 causal")
    assert ns > 1 and need > 0
    q, k, v = (upload(t, "f16") for t in (inp.q, inp.k, inp.v))
    o, lse = _outputs(inp)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def call(s):
        if noalloc:
            st = attn_fwd_splitkv_noalloc(q, k, v, o, lse, *args, s)
        else:
            st = attn_fwd_splitkv(q, k, v, o, lse, *args, ws, need, s)
        assert st == ATTN_OK

    _replays_match(call, (o, lse), label)
    _check_oracle(inp, o, lse, label)
