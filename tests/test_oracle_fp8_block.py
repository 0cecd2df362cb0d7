"""Pins of the block-scaled FP8 oracle (oracle/fp8_block.py), CPU only.

Each check takes the module under test, so the same checks run against the
oracle and against copies of it with planted mistakes (the mutation test at
the end), and each pins the module to something other than itself:

* the Walsh-Hadamard matrix against the closed form of its entries,
  (-1)^popcount(i & j) / 4, and against orthogonality;
* the transform against the identity the page states, (QH)(KH)^T = Q K^T,
  and against vectors whose transforms are known by hand;
* the E4M3 encoder exhaustively against the format's decoder (every finite
  code round-trips, every midpoint goes to the even code, saturation at 448)
  and against an independent grid-search encoder;
* block quantisation against its error bound, the amax code, block
  independence and the zero block;
* incoherent processing against the page's claim, qualitatively: on inputs
  with 0.1% outliers it lowers the error of FP8 attention against the exact
  result on the unquantised inputs (here by about 1.5x; the page reports
  2.6x on its own data).
"""

import importlib.util

import numpy as np
import pytest

import oracle
import oracle.fp8_block as fb_mod
from attention_forward_02_amd import inputs

E4M3_VALUES = oracle.decode_e4m3(np.arange(256))
FINITE = [c for c in range(256) if np.isfinite(E4M3_VALUES[c])]


def check_hadamard_closed_form(m):
    h = m.hadamard_matrix(16)
    i, j = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    parity = np.vectorize(lambda a: bin(a).count("1") & 1)(i & j)
    assert np.array_equal(h, np.where(parity == 1, -1.0, 1.0))
    x = np.eye(16)
    # row j of the identity transforms to column j of H / 4
    assert np.array_equal(m.hadamard16(x), np.where(parity == 1, -0.25, 0.25).T)
    hn = m.hadamard16(np.eye(16))
    assert np.allclose(hn @ hn.T, np.eye(16), atol=1e-15, rtol=0)


def check_hadamard_dot_products(m):
    rng = np.random.default_rng(7)
    for d in (64, 128, 256):
        q = rng.standard_normal((1, 2, 33, d))
        k = rng.standard_normal((1, 2, 47, d))
        s = q @ np.swapaxes(k, -1, -2)
        s2 = m.hadamard16(q) @ np.swapaxes(m.hadamard16(k), -1, -2)
        assert np.allclose(s2, s, rtol=0, atol=1e-12 * np.abs(s).max())
        # orthogonal and symmetric: applying it twice gives the input back
        assert np.allclose(m.hadamard16(m.hadamard16(q)), q, rtol=0, atol=1e-14)


def check_hadamard_special_vectors(m):
    x = np.zeros((1, 1, 1, 64))
    x[..., 16:32] = 3.0                         # a constant block
    x[..., 37] = 20.0                           # one spike in the third block
    y = m.hadamard16(x)[0, 0, 0]
    assert np.array_equal(y[:16], np.zeros(16))
    assert y[16] == 12.0 and np.array_equal(y[17:32], np.zeros(15))
    spike = np.array([20.0 / 4 * (-1) ** bin(i & 5).count("1") for i in range(16)])
    assert np.array_equal(y[32:48], spike)      # spread: every entry +-5
    assert np.array_equal(y[48:], np.zeros(16))


def check_encoder_round_trip(m):
    vals = E4M3_VALUES[FINITE]
    assert np.array_equal(m.encode_e4m3(vals), np.array(FINITE, dtype=np.uint8))


def check_encoder_midpoints(m):
    for c in range(0x7E):                      # consecutive positive codes c, c + 1
        lo, hi = E4M3_VALUES[c], E4M3_VALUES[c + 1]
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert m.encode_e4m3(np.array([mid]))[0] == even, (c, mid)
        assert m.encode_e4m3(np.array([np.nextafter(mid, np.inf)]))[0] == c + 1
        assert m.encode_e4m3(np.array([np.nextafter(mid, -np.inf)]))[0] == c
        assert m.encode_e4m3(np.array([-mid]))[0] == even | 0x80


def check_encoder_saturation(m):
    big = np.array([448.0, 448.5, 463.9, 464.0, 480.0, 1e6, -1e6, -450.0])
    assert list(m.encode_e4m3(big)) == [0x7E] * 6 + [0xFE] * 2


def check_encoder_matches_grid_search(m):
    rng = np.random.default_rng(11)
    y = (rng.standard_normal(200_000) * np.exp2(rng.uniform(-12, 10, 200_000))).astype(np.float32)
    assert np.array_equal(m.encode_e4m3(y), inputs.encode_e4m3(y))


def _outlier(shape, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape)
    hit = rng.random(shape) < 1e-3
    x[hit] *= 20.0
    return x


def check_quantize_bounds(m):
    x = _outlier((2, 3, 130, 128), 3)
    for had in (False, True):
        codes, ds = m.quantize_blocks(x, had)
        assert codes.shape == x.shape and ds.shape == (2, 3, 3) and ds.dtype == np.float32
        y = (m.hadamard16(x) if had else x).astype(np.float32).astype(np.float64)
        deq = m.dequantize_blocks(codes, ds)
        dsr = np.repeat(ds.astype(np.float64), [64, 64, 2], axis=2)[..., None]
        # half a code step: 2^-4 relative for normal codes, 2^-10 descales below
        bound = np.maximum(np.abs(y) * 2.0 ** -4, dsr * 2.0 ** -10) * (1 + 1e-6)
        assert np.all(np.abs(deq - y) <= bound)
        # the largest magnitude of every block maps to +-448
        for b in range(3):
            yb = y[:, :, 64 * b:64 * (b + 1)]
            cb = codes[:, :, 64 * b:64 * (b + 1)]
            flat_y = yb.reshape(6, -1)
            at = np.abs(flat_y).argmax(axis=1)
            picked = cb.reshape(6, -1)[np.arange(6), at]
            assert np.all((picked & 0x7F) == 0x7E)
            amax = np.abs(flat_y).max(axis=1)
            assert np.allclose(ds[:, :, b].reshape(6).astype(np.float64), amax / 448.0, rtol=2.0 ** -23, atol=0)


def check_quantize_blocks_independent(m):
    x = _outlier((1, 1, 200, 64), 4)
    c0, d0 = m.quantize_blocks(x, True)
    x2 = x.copy()
    x2[0, 0, 150, 5] = 1000.0                 # row 150: block 2 (rows 128..191)
    c1, d1 = m.quantize_blocks(x2, True)
    assert np.array_equal(c0[:, :, :128], c1[:, :, :128]) and np.array_equal(d0[..., :2], d1[..., :2])
    assert np.array_equal(c0[:, :, 192:], c1[:, :, 192:]) and d0[0, 0, 3] == d1[0, 0, 3]
    assert d1[0, 0, 2] > d0[0, 0, 2]
    z = np.zeros((1, 2, 70, 128))
    z[0, 1, 65, 3] = 2.0
    cz, dz = m.quantize_blocks(z, False)
    assert np.all(cz[0, 0] == 0) and np.all(dz[0, 0] == 1.0) and dz[0, 1, 0] == 1.0
    assert cz[0, 1, 65, 3] == 0x7E and dz[0, 1, 1] == np.float32(2.0) / np.float32(448.0)


def check_incoherent_processing_helps(m):
    # the FP8 workload's recipe: N(0, 1) entries, 0.1% of them times 20
    q, k, v = (_outlier((1, 8, 512, 128), seed) for seed in (5, 6, 7))
    scale = 1.0 / np.sqrt(128)
    o_ref, _ = oracle.attention(q, k, v, False, scale)

    def per_tensor(x):
        ds = np.float32(np.float32(np.abs(x).max()) / np.float32(448.0))
        return oracle.decode_e4m3(m.encode_e4m3((x.astype(np.float32) / ds).astype(np.float32))) * float(ds)

    def blocks(x, had):
        return m.dequantize_blocks(*m.quantize_blocks(x, had))

    def rel_rmse(qq, kk, vv):
        o, _ = oracle.attention(qq, kk, vv, False, scale)
        return np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref)

    naive = rel_rmse(per_tensor(q), per_tensor(k), per_tensor(v))
    smoothed = rel_rmse(blocks(q, True), blocks(k, True), blocks(v, False))
    assert smoothed < naive / 1.2, (naive, smoothed)


ALL_CHECKS = [check_hadamard_closed_form, check_hadamard_dot_products, check_hadamard_special_vectors,
              check_encoder_round_trip, check_encoder_midpoints, check_encoder_saturation,
              check_encoder_matches_grid_search, check_quantize_bounds, check_quantize_blocks_independent,
              check_incoherent_processing_helps]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_fp8_block_pins(check):
    check(fb_mod)


def test_fp8_block_imports():
    src = open(fb_mod.__file__).read()
    imports = [ln.strip() for ln in src.splitlines() if ln.startswith(("import ", "from "))]
    assert imports == ["import numpy as np", "from .forward import decode_e4m3"], imports


MUTANTS = [
    ("unnormalised transform", "_H16 = hadamard_matrix(16) / 4.0", "_H16 = hadamard_matrix(16) / 2.0"),
    ("wrong Sylvester sign", "h = np.block([[h, h], [h, -h]])", "h = np.block([[h, -h], [h, h]])"),
    ("transform rows not columns", "(blocks @ _H16.T)", "(_H16 @ blocks)"),
    ("truncating encoder", "value = np.rint(a / spacing) * spacing", "value = np.floor(a / spacing) * spacing"),
    ("ties away from zero", "value = np.rint(a / spacing) * spacing",
     "value = np.floor(a / spacing + 0.5) * spacing"),
    ("no saturation", "value = np.minimum(value, E4M3_MAX)", "value = value"),
    ("subnormal binade off", "binade = np.maximum(ex - 1, -6)", "binade = np.maximum(ex - 1, -7)"),
    ("exponent bias off", "e_field = np.where(sub, 0, vex - 1 + 7)", "e_field = np.where(sub, 0, vex + 7)"),
    ("FNUZ range", "E4M3_MAX = 448.0", "E4M3_MAX = 240.0"),
    ("block one row too long", "r0, r1 = blk * block_rows, min(N, (blk + 1) * block_rows)",
     "r0, r1 = blk * block_rows, min(N, (blk + 1) * block_rows + 1)"),
    ("per-tensor amax", "amax = np.abs(yb).max(axis=(2, 3))", "amax = np.abs(y32).max(axis=(2, 3))"),
    ("dequantise with the wrong block", "rows = np.arange(N) // block_rows", "rows = np.arange(N) // (block_rows * 2)"),
]


def _load_mutant(old, new):
    src = open(fb_mod.__file__).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    spec = importlib.util.spec_from_loader("oracle.fp8_block_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "oracle_fp8_block_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_fp8_block_pins_catch_planted_mistake(name, old, new):
    mod = _load_mutant(old, new)
    caught = []
    for check in ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError, OverflowError):
            caught.append(check.__name__)
    assert caught, f"no pin caught the planted mistake '{name}'"
