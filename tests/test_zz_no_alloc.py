"""The allocation-free split-key entry point (attn_fwd_splitkv_noalloc),
through the C ABI, against the entry point it mirrors (attn_fwd_splitkv on
a workspace allocated by the caller): bitwise-identical outputs, and both
within the stated tolerances of the float64 oracle.  Two calls in a row on
the device's static scratch, the second with a smaller input (fewer query
tiles, another head dim and format, causal), so the second call reuses
scratch left over by the first."""

import numpy as np
import pytest
import torch

from attention_forward_02_amd import inputs
from attention_forward_02_amd.binding import (ATTN_BF16, ATTN_F16, ATTN_OK, attn_fwd_splitkv, attn_fwd_splitkv_noalloc,
                                              attn_fwd_splitkv_num_splits, attn_fwd_splitkv_workspace_bytes)
from gpu_helpers import compare, dequant, oracle_all_heads, say, upload

pytestmark = pytest.mark.gpu

CODES = {"f16": ATTN_F16, "bf16": ATTN_BF16}


def _outputs(inp):
    dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float16
    o = torch.empty((inp.B, inp.H, inp.Nq, inp.d), dtype=dt, device="cuda")
    lse = torch.empty((inp.B, inp.H, inp.Nq), dtype=torch.float32, device="cuda")
    return o, lse


def _both(inp):
    q, k, v = (upload(t, inp.dtype) for t in (inp.q, inp.k, inp.v))
    args = (inp.B, inp.H, inp.Nq, inp.Nk, inp.d, inp.causal, float(inp.scale), CODES[inp.dtype], 1.0, 1.0, 1.0, 0)
    ns = attn_fwd_splitkv_num_splits(inp.B, inp.H, inp.Nq, inp.Nk, inp.d, inp.causal, CODES[inp.dtype], 0)
    need = attn_fwd_splitkv_workspace_bytes(inp.B, inp.H, inp.Nq, inp.Nk, inp.d, inp.causal, CODES[inp.dtype], 0)
    say(f"[gpu] noalloc vs workspace: B={inp.B} H={inp.H} Nq={inp.Nq} Nk={inp.Nk} d={inp.d} {inp.dtype} "
        f"causal={inp.causal}: {ns} splits, {need} bytes of partials")
    assert ns > 1 and 0 < need
    o1, l1 = _outputs(inp)
    assert attn_fwd_splitkv_noalloc(q, k, v, o1, l1, *args) == ATTN_OK
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o2, l2 = _outputs(inp)
    assert attn_fwd_splitkv(q, k, v, o2, l2, *args, ws, need) == ATTN_OK
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2), \
        "the allocation-free entry point differs from the workspace one"
    qq, kk, vv = dequant(inp)
    o_ref, l_ref = oracle_all_heads(qq, kk, vv, inp.causal, float(inp.scale))
    stats = compare(o1.view(torch.int16).cpu().numpy().view(np.uint16), l1.cpu().numpy(), o_ref, l_ref, inp.dtype,
                    "noalloc")
    say(f"[gpu] noalloc: {stats}")


def test_noalloc_matches_workspace_entry_point_twice():
    _both(inputs.make(1, 8, 256, 16384, 128, "f16", seed=71))
    _both(inputs.make(1, 2, 100, 3000, 64, "bf16", seed=72, causal=True))
