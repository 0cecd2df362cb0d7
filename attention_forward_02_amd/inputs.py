"""Seeded synthetic inputs for the attention forward workloads.

Used by the tests, the benchmark and the smoke check.  This module draws
random numbers and encodes them into the element formats the library reads
(IEEE binary16, bfloat16, OCP FP8 E4M3 with a per-tensor descale).  It holds
none of the forward pass's arithmetic, imports only NumPy, and is the only
code that both the HIP path's callers and the CPU oracle's callers share.

Workloads (all inputs i.i.d. N(0, 1) float32, scale = fp32(1/sqrt(d))):

==========================  ==  ==  =====  =====  ===  ======  =====
name                        B   H   Nq     Nk     d    causal  dtype
==========================  ==  ==  =====  =====  ===  ======  =====
tiny_d64_f16                1   1   128    128    64   no      f16
causal_d64_bf16             4   8   1024   1024   64   yes     bf16
hd128_seq8k_f16             2   16  8192   8192   128  no      f16
causal_d256_bf16            1   16  16384  16384  256  yes     bf16
hd128_seq8k_e4m3            2   16  8192   8192   128  no      e4m3
hd128_seq8k_e4m3_smoothed   2   16  8192   8192   128  no      f16
==========================  ==  ==  =====  =====  ===  ======  =====

``hd128_seq8k_f16`` is the head-dim-128, sequence-8192 FP16 shape of the
pingpong measurement reported for FlashAttention-3 (Warp-specialization
concept card, "Pingpong scheduling between two consumer warpgroups").  The
e4m3 workload adds 0.1% outliers (entries multiplied by 20) to every tensor
before per-tensor quantisation, the situation the FP8 section of "Inside
FlashAttention-3" (section 5) targets.  ``hd128_seq8k_e4m3_smoothed``
draws the same float32 values (same seed) but hands them over as binary16:
its path quantises them on the GPU itself, block-scaled, with Q and K
Walsh-Hadamard-smoothed first (the second FP8 item of that section).
"""

from dataclasses import dataclass, field
import math

import numpy as np

DTYPES = ("f16", "bf16", "e4m3")

WORKLOADS = {
    "tiny_d64_f16": dict(B=1, H=1, Nq=128, Nk=128, d=64, causal=False, dtype="f16", seed=1001),
    "causal_d64_bf16": dict(B=4, H=8, Nq=1024, Nk=1024, d=64, causal=True, dtype="bf16", seed=1002),
    "hd128_seq8k_f16": dict(B=2, H=16, Nq=8192, Nk=8192, d=128, causal=False, dtype="f16", seed=1003),
    "causal_d256_bf16": dict(B=1, H=16, Nq=16384, Nk=16384, d=256, causal=True, dtype="bf16", seed=1004),
    "hd128_seq8k_e4m3": dict(B=2, H=16, Nq=8192, Nk=8192, d=128, causal=False, dtype="e4m3",
                             seed=1005, outliers=True),
    "hd128_seq8k_e4m3_smoothed": dict(B=2, H=16, Nq=8192, Nk=8192, d=128, causal=False, dtype="f16",
                                      seed=1005, outliers=True, smoothed=True),
}

E4M3_MAX = 448.0
OUTLIER_RATE = 1e-3
OUTLIER_GAIN = 20.0
# Score rise (natural units) between consecutive key ranges of the
# ``stairs`` recipe: 8 > 8 ln 2, so in base 2 each rise exceeds 8 plus the
# spread of a 64-key tile maximum.
STAIR_HEIGHT = 8.0


# ---------------------------------------------------------------------------
# Encoders: float32 -> element codes, round to nearest even
# ---------------------------------------------------------------------------

def encode_f16(x):
    """float32 -> IEEE binary16 codes (uint16), round to nearest even."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def encode_bf16(x):
    """float32 -> bfloat16 codes (uint16), round to nearest even on the low
    16 bits of the binary32 pattern.  Inputs here are always finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def _e4m3_grid():
    """All non-negative finite E4M3 values, indexed by their code 0..126."""
    codes = np.arange(127)
    e = codes >> 3
    m = (codes & 7).astype(np.float64)
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))


_E4M3_GRID = _e4m3_grid()


def encode_e4m3(y):
    """float -> OCP E4M3 codes (uint8): round to nearest, ties to the even
    code, magnitudes beyond 448 saturate to +-448 (code 0x7E / 0xFE)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), E4M3_MAX)
    hi = np.searchsorted(_E4M3_GRID, a, side="left")        # first grid >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_GRID[lo]
    d_hi = _E4M3_GRID[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(y), code | 0x80, code).astype(np.uint8)


# ---------------------------------------------------------------------------
# Inputs
# ---------------------------------------------------------------------------

@dataclass
class Inputs:
    """One attention call's inputs, as the bits a GPU receives.

    q, k, v: [B, H, N, d] arrays of element codes (uint16 for f16/bf16, uint8
    for e4m3).  ``scale`` multiplies Q K^T; ``descale`` gives each tensor's
    per-tensor dequantisation factor (1.0 unless dtype is e4m3).  ``q32`` etc.
    hold the float32 values before encoding.
    """
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    dtype: str
    scale: np.float32
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    descale: tuple = (np.float32(1.0), np.float32(1.0), np.float32(1.0))
    q32: np.ndarray = field(default=None, repr=False)
    k32: np.ndarray = field(default=None, repr=False)
    v32: np.ndarray = field(default=None, repr=False)


def default_scale(d):
    """fp32(1/sqrt(d)), computed in float64 and rounded once."""
    return np.float32(1.0 / math.sqrt(d))


def _draw(rng, shape, outliers):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if outliers:
        hit = rng.random(size=shape) < OUTLIER_RATE
        x[hit] *= np.float32(OUTLIER_GAIN)
    return x


def make(B, H, Nq, Nk, d, dtype, seed, causal=False, outliers=False, scale=None, keep_f32=False, kgrow=0.0,
         stairs=0, outlier_tensors="qkv"):
    """Draw Q, K, V (in that order) from ``numpy.random.default_rng(seed)``
    and encode them as ``dtype``.  For e4m3 each tensor gets descale =
    fp32(amax / 448) and codes = RNE-saturate(x / descale).

    ``outlier_tensors`` names the tensors that get outliers (default all
    three).

    Two recipes make a row's maximum score arrive many key tiles after its
    first, so that the running row max of the online softmax rises by large
    steps during the key loop:
    * ``kgrow`` > 0 multiplies key row j by 1 + kgrow * j / Nk (in float32,
      before encoding): scores grow gradually along the key axis;
    * ``stairs`` = n > 0 sets channel 0 of every query row to 1 and channel 0
      of key row j to STAIR_HEIGHT * floor((n + 1) j / Nk) / scale, so that
      the scores of the (i+1)-th of n + 1 equal key ranges are raised by
      i * STAIR_HEIGHT (natural units) over the first range's, while inside
      a range they spread as in the plain workload."""
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.default_rng(seed)
    q32 = _draw(rng, (B, H, Nq, d), outliers and "q" in outlier_tensors)
    k32 = _draw(rng, (B, H, Nk, d), outliers and "k" in outlier_tensors)
    v32 = _draw(rng, (B, H, Nk, d), outliers and "v" in outlier_tensors)
    sc = default_scale(d) if scale is None else np.float32(scale)
    if kgrow:
        g = (1.0 + float(kgrow) * np.arange(Nk, dtype=np.float64) / Nk).astype(np.float32)
        k32 = k32 * g[None, None, :, None]
    if stairs:
        step = np.floor((stairs + 1) * np.arange(Nk, dtype=np.float64) / Nk)
        q32[..., 0] = 1.0
        k32[..., 0] = (STAIR_HEIGHT * step / float(sc)).astype(np.float32)[None, None, :]
    desc = (np.float32(1.0),) * 3
    if dtype == "f16":
        q, k, v = encode_f16(q32), encode_f16(k32), encode_f16(v32)
    elif dtype == "bf16":
        q, k, v = encode_bf16(q32), encode_bf16(k32), encode_bf16(v32)
    else:
        enc = []
        desc = []
        for x in (q32, k32, v32):
            amax = float(np.abs(x).max()) if x.size else 1.0
            ds = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
            desc.append(ds)
            enc.append(encode_e4m3(x.astype(np.float64) / np.float64(ds)))
        q, k, v = enc
        desc = tuple(desc)
    out = Inputs(B=B, H=H, Nq=Nq, Nk=Nk, d=d, causal=bool(causal), dtype=dtype, scale=sc,
                 q=q, k=k, v=v, descale=desc)
    if keep_f32:
        out.q32, out.k32, out.v32 = q32, k32, v32
    return out


def make_workload(name, keep_f32=False):
    """Inputs of one named workload (see the table in the module docstring)."""
    w = dict(WORKLOADS[name])
    return make(w["B"], w["H"], w["Nq"], w["Nk"], w["d"], w["dtype"], w["seed"],
                causal=w["causal"], outliers=w.get("outliers", False), keep_f32=keep_f32)


def flops(B, H, Nq, Nk, d, causal):
    """Attention forward FLOPs as the pages count them: 4*B*H*Nq*Nk*d (two
    matrix products of 2*Nq*Nk*d each), halved when causal."""
    f = 4.0 * B * H * Nq * Nk * d
    return f / 2.0 if causal else f
