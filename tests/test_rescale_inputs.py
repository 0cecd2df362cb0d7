"""CPU checks of the rescale-forcing inputs used by tests/test_rescale_gpu.py.

* Every recipe, head dim, format and causality forces the lazy online-softmax
  reference to be raised for several rows (so the rescale
  branch of every kernel runs); the staircase recipe also in the second half
  of the key range alone, which the split-key kernel's second wave group
  walks with a reference of its own.
* The cases are sensitive to the rescale factor: the oracle's own blockwise
  loop with the output rescale left out, or with the inverse factor (the
  mistake the concept card corrects below its sketch), misses the 4e-3 gate
  by orders of magnitude on these inputs, so a kernel with either mistake
  cannot pass them.
"""

import importlib.util

import numpy as np
import pytest

from oracle import forward as oracle_mod
from attention_forward_02_amd import inputs
from gpu_helpers import dequant, rescales_from_inputs

RECIPES = {
    "stairs": dict(stairs=3),
    "late": dict(kgrow=3.0),
    "scale1": dict(scale=1.0),
    "outliers": dict(outliers=True, outlier_tensors="qk"),
}
N = 520


@pytest.mark.parametrize("recipe", list(RECIPES))
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_recipes_force_the_rescale(d, dtype, causal, recipe):
    for seed in (500 + d, 507 + d):
        inp = inputs.make(1, 2, N, N, d, dtype, seed=seed + int(causal), causal=causal, **RECIPES[recipe])
        q, k, _ = dequant(inp)
        first = rescales_from_inputs(q, k, float(inp.scale), causal)
        assert (first > 0).sum() >= 8
        if recipe == "stairs":
            second = rescales_from_inputs(q, k, float(inp.scale), causal, start_tile=5)
            assert (second > 0).sum() >= 32


def test_plain_workload_never_rescales():
    # the reason these recipes exist: N(0, 1) inputs at 1/sqrt(d) stay below
    # the lazy threshold after the first tile
    inp = inputs.make(1, 2, N, N, 128, "f16", seed=3)
    q, k, _ = dequant(inp)
    assert rescales_from_inputs(q, k, float(inp.scale), False).sum() == 0


def _mutant(old, new):
    src = open(oracle_mod.__file__).read()
    assert src.count(old) == 1, f"mutation anchor not found: {old!r}"
    spec = importlib.util.spec_from_loader("oracle_rescale_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src.replace(old, new), "oracle_rescale_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("old,new", [
    ("output = factor[:, None] * output + probs @ v[b, h, j0:j1]", "output = output + probs @ v[b, h, j0:j1]"),
    ("factor = np.exp(row_max - ref)", "factor = np.exp(ref - row_max)"),
])
@pytest.mark.parametrize("recipe", list(RECIPES))
def test_rescale_mistakes_miss_the_gate(recipe, old, new):
    inp = inputs.make(1, 1, 256, N, 64, "f16", seed=11, **RECIPES[recipe])
    q, k, v = dequant(inp)
    scale = float(inp.scale)
    o_ref, _ = oracle_mod.attention(q, k, v, False, scale)
    with np.errstate(all="ignore"):
        o_bad, _ = _mutant(old, new).attention_blockwise(q, k, v, False, scale, 64)
    err = np.nan_to_num(np.abs(o_bad - o_ref), nan=np.inf).max()
    assert err > 100 * 4e-3
