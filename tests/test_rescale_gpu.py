"""The online-softmax rescale on every 16-bit kernel, against the oracle.

When a later key tile raises a row's maximum, the running output and row
sum are multiplied by exp(old max - new max), the factor the concept card
gives below its implementation sketch.  The kernels raise their reference
lazily (only when a row max rises by more than 8 in base 2), so inputs
drawn like the benchmark workloads -- N(0, 1) at scale 1/sqrt(d) -- never
take that branch after the first tile.  These inputs do, on purpose:

* ``stairs``: the scores of four equal key ranges are raised in steps of 8
  (natural units), so each range's first tile rescales a nonzero output by
  about 2^-11.5, while inside a range the scores spread as in the
  benchmark;
* ``late``: key row j scaled by 1 + 3 j / Nk, so the row maximum keeps
  rising along the key axis;
* ``scale1``: scale = 1 instead of 1/sqrt(d);
* ``outliers``: 0.1% of the entries of Q and K multiplied by 20 (V stays
  N(0, 1), so |O| stays in the range where fp16 rounds below 4e-3).

Each case first checks on the inputs (gpu_helpers.rescales_from_inputs)
that the branch must be taken (for the staircase also in the second half of
the key range alone, which the split-key kernel's second wave group walks
with a reference of its own), then compares every output with the oracle.  binary16 is gated at the stated 4e-3; bfloat16 at
4e-3 + half an output ulp, and on the peaked recipes (late, scale1,
outliers) also plus 2^-9 (P |V|), its rounding of P (tests/gpu_helpers.py).
"""

import numpy as np
import pytest
import torch

from attention_forward_02_amd import VARIANT_NAMES, attention, attn_variant_available, inputs
from attention_forward_02_amd.binding import ATTN_BF16, ATTN_F16
from gpu_helpers import compare, dequant, oracle_all_heads, rescales_from_inputs, say, upload

pytestmark = pytest.mark.gpu

CODES = {"f16": ATTN_F16, "bf16": ATTN_BF16}
KERNELS = [(d, dt, var) for d in (64, 128, 256) for dt in ("f16", "bf16") for var in range(len(VARIANT_NAMES))
           if attn_variant_available(d, CODES[dt], var)]
RECIPES = {
    "stairs": dict(stairs=3),
    "late": dict(kgrow=3.0),
    "scale1": dict(scale=1.0),
    "outliers": dict(outliers=True, outlier_tensors="qk"),
}
N = 520  # eight full 64-key tiles and a ragged ninth


@pytest.mark.parametrize("recipe", list(RECIPES))
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,dtype,variant", KERNELS, ids=[f"d{d}-{t}-{VARIANT_NAMES[v]}" for d, t, v in KERNELS])
def test_rescale_parity(d, dtype, variant, causal, recipe):
    label = f"rescale {recipe} {VARIANT_NAMES[variant]} d={d} {dtype} causal={causal}"
    say(f"[gpu] {label}: B=1 H=2 N={N}")
    inp = inputs.make(1, 2, N, N, d, dtype, seed=500 + d + 3 * variant + int(causal), causal=causal,
                      **RECIPES[recipe])
    q64, k64, v64 = dequant(inp)
    scale = float(inp.scale)
    first = rescales_from_inputs(q64, k64, scale, causal)
    assert (first > 0).sum() >= 8, f"{label}: inputs do not force the rescale"
    if recipe == "stairs":
        second = rescales_from_inputs(q64, k64, scale, causal, start_tile=(-(-N // 64) + 1) // 2)
        assert (second > 0).sum() >= 32, f"{label}: inputs do not force the rescale in the second key half"
    q, k, v = (upload(t, dtype) for t in (inp.q, inp.k, inp.v))
    o, lse = attention(q, k, v, causal=causal, scale=scale, variant=variant or None)
    torch.cuda.synchronize()
    o_codes = o.view(torch.int16).cpu().numpy().view(np.uint16)
    o_ref, lse_ref = oracle_all_heads(q64, k64, v64, causal, scale)
    p_abs_v = None
    if dtype == "bf16" and recipe != "stairs":
        p_abs_v, _ = oracle_all_heads(q64, k64, np.abs(v64), causal, scale)
    stats = compare(o_codes, lse.cpu().numpy(), o_ref, lse_ref, dtype, label, p_abs_v=p_abs_v)
    say(f"[gpu] {label}: {stats}; rows that rescale: {int((first > 0).sum())}")
