"""Pins for the float64 oracle, all on the CPU.

Each ``check_*`` function takes the oracle module so that the mutation test at
the bottom can run the same pins against deliberately broken copies of it and
show that every planted mistake is caught by at least one pin.

Pins used (none of them re-types the oracle's own formula):
* hand-derived closed forms in tests/golden/closed_forms.json;
* torch's float64 CPU scaled_dot_product_attention and logsumexp (an
  independent library implementation of the same definition);
* invariants the definition implies: V = 1 gives O = 1; Q = 0 gives the mean
  (causal: prefix mean) of V and LSE = ln(#keys); V = identity makes O the
  probability matrix, whose rows sum to 1; shifting every score of a row by a
  constant moves LSE by it and leaves O alone; permuting keys with their
  values changes nothing; one key gives O = v0; a huge scale gives hard
  attention;
* a pure-Python brute force with math.fsum on tiny inputs;
* the blockwise online-softmax variant against the two-pass definition;
* the decoders against torch's own dtype casts on every code.
"""

import importlib.util
import json
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import forward as oracle_mod

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------------------
# check functions (module under test passed in)
# ---------------------------------------------------------------------------

def check_golden(mod):
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        q = np.array(c["q"], dtype=np.float64)[None, None]
        k = np.array(c["k"], dtype=np.float64)[None, None]
        v = np.array(c["v"], dtype=np.float64)[None, None]
        for key, causal in (("noncausal", False), ("causal", True)):
            if key not in c:
                continue
            exp_o = np.array(c[key]["o"], dtype=np.float64)
            exp_l = np.array([float(x) for x in c[key]["lse"]], dtype=np.float64)
            o, l = mod.attention(q, k, v, causal, c["scale"])
            np.testing.assert_allclose(o[0, 0], exp_o, rtol=1e-14, atol=1e-14, err_msg=c["name"])
            np.testing.assert_array_equal(np.isinf(l[0, 0]), np.isinf(exp_l))
            fin = np.isfinite(exp_l)
            np.testing.assert_allclose(l[0, 0][fin], exp_l[fin], rtol=1e-14, atol=1e-14, err_msg=c["name"])


def _torch_reference(q, k, v, causal, scale):
    """torch float64 CPU attention with a bottom-right causal mask."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    Nq, Nk = q.shape[2], k.shape[2]
    mask = None
    if causal:
        i = torch.arange(Nq)[:, None]
        j = torch.arange(Nk)[None, :]
        mask = j <= i + (Nk - Nq)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    s = scale * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
    if mask is not None:
        s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy()


def check_torch(mod):
    rng = np.random.default_rng(5)
    for (B, H, Nq, Nk, d, dv, causal) in [(2, 3, 17, 17, 8, 8, False), (1, 2, 33, 33, 16, 4, True),
                                          (2, 1, 9, 23, 8, 8, True), (1, 1, 40, 7, 4, 5, False)]:
        q, k, v = _rand(rng, B, H, Nq, d), _rand(rng, B, H, Nk, d), _rand(rng, B, H, Nk, dv)
        scale = 0.7
        o, l = mod.attention(q, k, v, causal, scale)
        ro, rl = _torch_reference(q, k, v, causal, scale)
        np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(l, rl, rtol=1e-12, atol=1e-12)


def check_invariants(mod):
    rng = np.random.default_rng(11)
    B, H, N, d = 2, 2, 19, 8
    q, k = _rand(rng, B, H, N, d), _rand(rng, B, H, N, d)
    v = _rand(rng, B, H, N, d)
    scale = 1.0 / math.sqrt(d)
    for causal in (False, True):
        # V = 1 gives O = 1
        o, _ = mod.attention(q, k, np.ones_like(v), causal, scale)
        np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-13)
        # Q = 0: O is the mean (causal: prefix mean) of V, LSE = ln(#keys)
        o, l = mod.attention(np.zeros_like(q), k, v, causal, scale)
        if causal:
            n = np.arange(1, N + 1, dtype=np.float64)
            mean = np.cumsum(v, axis=2) / n[None, None, :, None]
        else:
            n = np.full(N, float(N))
            mean = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        np.testing.assert_allclose(o, mean, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(l, np.broadcast_to(np.log(n), l.shape), rtol=1e-14, atol=1e-14)
        # V = identity: O = P; rows sum to 1, masked entries are 0
        eye = np.broadcast_to(np.eye(N), (B, H, N, N))
        p, _ = mod.attention(q, k, eye, causal, scale)
        np.testing.assert_allclose(p.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
        assert (p >= 0).all()
        if causal:
            assert np.all(p[..., np.triu_indices(N, 1)[0], np.triu_indices(N, 1)[1]] == 0.0)
            # row 0 sees key 0 only: O0 = V0 and LSE0 = S00
            o, l = mod.attention(q, k, v, True, scale)
            np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], rtol=1e-14, atol=1e-14)
            s00 = scale * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0])
            np.testing.assert_allclose(l[:, :, 0], s00, rtol=1e-13, atol=1e-13)
        # shift: extra column a in Q and 1 in K moves every score by scale*a
        a = 1.7
        q2 = np.concatenate([q, np.full(q.shape[:3] + (1,), a)], axis=-1)
        k2 = np.concatenate([k, np.ones(k.shape[:3] + (1,))], axis=-1)
        o1, l1 = mod.attention(q, k, v, causal, scale)
        o2, l2 = mod.attention(q2, k2, v, causal, scale)
        np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(l2, l1 + scale * a, rtol=1e-12, atol=1e-12)
    # joint key/value permutation leaves the non-causal result unchanged
    perm = rng.permutation(N)
    o1, l1 = mod.attention(q, k, v, False, scale)
    o2, l2 = mod.attention(q, k[:, :, perm], v[:, :, perm], False, scale)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-12)
    # one key: O = v0, LSE = s0
    o, l = mod.attention(q, k[:, :, :1], v[:, :, :1], False, scale)
    np.testing.assert_allclose(o, np.broadcast_to(v[:, :, :1], o.shape), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(l, scale * np.einsum("bhnd,bhd->bhn", q, k[:, :, 0]), rtol=1e-13, atol=1e-13)
    # hard attention as the scale grows: O -> V[argmax score]
    big = 1e4
    o, _ = mod.attention(q, k, v, False, big)
    am = np.argmax(np.einsum("bhid,bhjd->bhij", q, k), axis=-1)
    hard = np.take_along_axis(v, am[..., None], axis=2)
    np.testing.assert_allclose(o, hard, rtol=0, atol=1e-9)


def _brute(q, k, v, causal, scale):
    """Pure-Python loops over one (b, h) pair; math.exp/fsum/log."""
    Nq, d = len(q), len(q[0])
    Nk, dv = len(k), len(v[0])
    O, L = [], []
    for i in range(Nq):
        s = []
        for j in range(Nk):
            if causal and j > i + (Nk - Nq):
                continue
            s.append((j, scale * math.fsum(q[i][c] * k[j][c] for c in range(d))))
        if not s:
            O.append([0.0] * dv)
            L.append(-math.inf)
            continue
        m = max(x for _, x in s)
        w = [(j, math.exp(x - m)) for j, x in s]
        tot = math.fsum(e for _, e in w)
        O.append([math.fsum(e * v[j][c] for j, e in w) / tot for c in range(dv)])
        L.append(m + math.log(tot))
    return O, L


def check_brute(mod):
    rng = np.random.default_rng(3)
    for (Nq, Nk, d, dv) in [(1, 1, 1, 1), (3, 5, 4, 2), (5, 3, 2, 3), (8, 8, 8, 8), (6, 6, 3, 1)]:
        q, k, v = _rand(rng, 1, 1, Nq, d), _rand(rng, 1, 1, Nk, d), _rand(rng, 1, 1, Nk, dv)
        for causal in (False, True):
            o, l = mod.attention(q, k, v, causal, 0.9)
            bo, bl = _brute(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), causal, 0.9)
            np.testing.assert_allclose(o[0, 0], np.array(bo), rtol=1e-13, atol=1e-14)
            bl = np.array(bl)
            np.testing.assert_array_equal(np.isinf(l[0, 0]), np.isinf(bl))
            np.testing.assert_allclose(l[0, 0][np.isfinite(bl)], bl[np.isfinite(bl)], rtol=1e-13, atol=1e-14)


def check_rows_subset(mod):
    rng = np.random.default_rng(8)
    q, k, v = _rand(rng, 1, 2, 40, 8), _rand(rng, 1, 2, 50, 8), _rand(rng, 1, 2, 50, 8)
    rows = np.array([0, 3, 17, 39])
    for causal in (False, True):
        o, l = mod.attention(q, k, v, causal, 0.5)
        os_, ls_ = mod.attention(q, k, v, causal, 0.5, rows=rows, row_chunk=3)
        np.testing.assert_allclose(os_, o[:, :, rows], rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(ls_, l[:, :, rows], rtol=1e-14, atol=1e-14)


def check_blockwise(mod):
    rng = np.random.default_rng(21)
    for (Nq, Nk, causal) in [(37, 37, False), (37, 37, True), (20, 45, True), (45, 20, True), (64, 130, False)]:
        q, k, v = _rand(rng, 1, 2, Nq, 16), _rand(rng, 1, 2, Nk, 16), _rand(rng, 1, 2, Nk, 16)
        o, l = mod.attention(q, k, v, causal, 0.25)
        for block in (1, 3, 16, 64, 128, Nk):
            ob, lb = mod.attention_blockwise(q, k, v, causal, 0.25, block)
            np.testing.assert_allclose(ob, o, rtol=1e-12, atol=1e-12)
            np.testing.assert_array_equal(np.isinf(lb), np.isinf(l))
            fin = np.isfinite(l)
            np.testing.assert_allclose(lb[fin], l[fin], rtol=1e-12, atol=1e-12)


def check_blockwise_golden(mod):
    for c in json.load(open(GOLDEN))["cases"]:
        q = np.array(c["q"], dtype=np.float64)[None, None]
        k = np.array(c["k"], dtype=np.float64)[None, None]
        v = np.array(c["v"], dtype=np.float64)[None, None]
        for key, causal in (("noncausal", False), ("causal", True)):
            if key not in c:
                continue
            o, _ = mod.attention_blockwise(q, k, v, causal, c["scale"], 1)
            np.testing.assert_allclose(o[0, 0], np.array(c[key]["o"]), rtol=1e-13, atol=1e-13)


def _torch_decode(codes, tdtype):
    t = torch.from_numpy(codes.view(np.int16) if codes.dtype == np.uint16 else codes)
    return t.view(tdtype).to(torch.float64).numpy()


def check_decoders(mod):
    codes16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for fn, td in ((mod.decode_f16, torch.float16), (mod.decode_bf16, torch.bfloat16)):
        ours, ref = fn(codes16), _torch_decode(codes16, td)
        np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
        ok = ~np.isnan(ref)
        np.testing.assert_array_equal(ours[ok], ref[ok])
    codes8 = np.arange(256, dtype=np.uint8)
    ours, ref = mod.decode_e4m3(codes8), _torch_decode(codes8, torch.float8_e4m3fn)
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])
    # format facts: max finite 448, min subnormal 2^-9, NaN only at 0x7F/0xFF
    assert mod.decode_e4m3(np.array([0x7E]))[0] == 448.0
    assert mod.decode_e4m3(np.array([0x01]))[0] == 2.0 ** -9
    assert np.isnan(mod.decode_e4m3(np.array([0x7F, 0xFF]))).all()
    assert mod.decode_f16(np.array([0x3C00]))[0] == 1.0
    assert mod.decode_bf16(np.array([0x3F80]))[0] == 1.0


ALL_CHECKS = [check_golden, check_torch, check_invariants, check_brute, check_rows_subset,
              check_blockwise, check_blockwise_golden, check_decoders]


# ---------------------------------------------------------------------------
# tests on the real oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pins(check):
    check(oracle_mod)


def test_package_exports():
    for name in ("attention", "attention_blockwise", "decode_f16", "decode_bf16", "decode_e4m3"):
        assert getattr(oracle, name) is getattr(oracle_mod, name)


def test_oracle_imports_nothing_of_the_product():
    src = open(oracle_mod.__file__).read()
    imports = [ln.strip() for ln in src.splitlines() if ln.startswith(("import ", "from "))]
    assert imports == ["import math", "import numpy as np"], imports


# ---------------------------------------------------------------------------
# mutation test: plant plausible mistakes in copies of the oracle (CPU only)
# ---------------------------------------------------------------------------

MUTANTS = [
    ("dropped scale", "s = scale * (q[b, h, r] @ kt)", "s = (q[b, h, r] @ kt)"),
    ("strict causal mask", "keys[None, :] <= rows[:, None] + (Nk - Nq)", "keys[None, :] < rows[:, None] + (Nk - Nq)"),
    ("top-left causal alignment", "keys[None, :] <= rows[:, None] + (Nk - Nq)", "keys[None, :] <= rows[:, None]"),
    ("inverted mask alignment sign", "rows[:, None] + (Nk - Nq)", "rows[:, None] + (Nq - Nk)"),
    ("LSE without the max", "m_ref + np.log(safe_l)", "np.log(safe_l)"),
    ("no normalisation", "o / safe_l[:, None]", "o"),
    ("values reversed", "o = p @ vb", "o = p @ vb[::-1]"),
    ("keys reversed", "kt = k[b, h].T", "kt = k[b, h][::-1].T"),
    ("inverse rescale factor", "factor = np.exp(row_max - ref)", "factor = np.exp(ref - row_max)"),
    ("rescale only the sum", "output = factor[:, None] * output + probs @ v[b, h, j0:j1]",
     "output = output + probs @ v[b, h, j0:j1]"),
    ("blockwise LSE base 2", "lse[b, h] = np.where(has_key, row_max + np.log(safe), -np.inf)",
     "lse[b, h] = np.where(has_key, row_max + np.log2(safe), -np.inf)"),
    ("exponent bias off by one", "np.exp2((e - bias).astype(np.float64))", "np.exp2((e - bias + 1).astype(np.float64))"),
    ("subnormal scale", "math.ldexp(1.0, 1 - bias)", "math.ldexp(1.0, -bias)"),
    ("fn NaN rule dropped", "nan = (e == emax) & (m == (1 << man_bits) - 1)", "nan = (e == emax) & (m < 0)"),
    ("empty rows give NaN", "np.where(has_key[:, None], o / safe_l[:, None], 0.0)", "o / l[:, None]"),
]


def _load_mutant(old, new):
    src = open(oracle_mod.__file__).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new)
    spec = importlib.util.spec_from_loader("oracle_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new):
    mod = _load_mutant(old, new)
    caught = []
    for check in ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(check.__name__)
    assert caught, f"no pin caught the planted mistake '{name}'"
