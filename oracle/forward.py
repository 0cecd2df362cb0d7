"""Float64 CPU oracle for the fused attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it.  It shares no code with the HIP library (no kernels, headers, helpers,
tables or pre/post-processing) and imports nothing but NumPy and ``math``.

What it computes (sources are the web pages on warp-specialised attention):

* ``attention`` is the plain definition of the forward pass that every page
  is about: scores S = scale * Q K^T, a softmax over each row of S, the output
  O = P V and the per-row log-sum-exp LSE = m + log(sum exp(S - m)).  The
  Warp-specialization concept card ("Implementation sketch", the consumer
  role) returns exactly ``(O / row_sum, row_max + log(row_sum))``; its note
  under the sketch says that pingpong and the in-warpgroup overlap change the
  schedule, never the result, so the oracle is the definition written out,
  in two passes (row max, then exp / sum / weighted sum of V).
* ``attention_blockwise`` follows the consumer loop of the same sketch step by
  step: per key block, a new running max, probabilities relative to it, the
  running sum rescaled by exp(old max - new max), the output rescaled by the
  same factor (the corrected factor the card states below its sketch), and at
  the end output / sum and max + log(sum).  It exists to pin the online
  softmax algebra against the two-pass definition.
* ``decode_f16`` / ``decode_bf16`` / ``decode_e4m3`` turn the exact bits that
  a GPU receives into float64, from the IEEE-754 binary16, bfloat16 and OCP
  FP8 E4M3 ("fn": no infinities, only S.1111.111 is NaN, max 448) format
  definitions.  FP8 E4M3 inputs with per-tensor scaling are the low-precision
  variant of the forward pass on the "Inside FlashAttention-3" page (section 5).

Readings where the pages are silent (each is listed in the design notes):

* the scale multiplies Q K^T before the max (the sketch has no scale; the
  definition softmax(Q K^T * scale) fixes it);
* LSE is in natural log;
* causal masking keeps key j for query i iff j <= i + (Nk - Nq) (bottom-right
  alignment; equals j <= i when Nq == Nk);
* a row with no allowed key has O = 0 and LSE = -inf.

Parity status: every function here is pinned by the CPU tests (brute force on
tiny inputs, closed forms, invariants, torch's float64 attention, exhaustive
codec tables); none is "parity unpinned".
"""

import math

import numpy as np

__all__ = [
    "decode_f16",
    "decode_bf16",
    "decode_e4m3",
    "attention",
    "attention_blockwise",
    "causal_allowed",
]


# ---------------------------------------------------------------------------
# Bit-exact decoders (format definitions, not library casts)
# ---------------------------------------------------------------------------

def _decode_binary(bits, exp_bits, man_bits, bias, fn_nan):
    """Decode an unsigned integer array of sign|exponent|mantissa codes.

    ``fn_nan`` selects the OCP "fn" convention (no infinities; only the code
    with all exponent and mantissa bits set is NaN) instead of IEEE-754
    (exponent all ones: infinity when the mantissa is 0, NaN otherwise).
    """
    b = np.asarray(bits).astype(np.int64)
    sign = np.where((b >> (exp_bits + man_bits)) & 1, -1.0, 1.0)
    e = (b >> man_bits) & ((1 << exp_bits) - 1)
    m = (b & ((1 << man_bits) - 1)).astype(np.float64)
    emax = (1 << exp_bits) - 1
    frac = m / float(1 << man_bits)
    normal = sign * (1.0 + frac) * np.exp2((e - bias).astype(np.float64))
    sub = sign * frac * math.ldexp(1.0, 1 - bias)
    out = np.where(e == 0, sub, normal)
    if fn_nan:
        nan = (e == emax) & (m == (1 << man_bits) - 1)
        out = np.where(nan, np.nan, out)
    else:
        out = np.where((e == emax) & (m == 0), sign * np.inf, out)
        out = np.where((e == emax) & (m != 0), np.nan, out)
    return out


def decode_f16(bits):
    """IEEE-754 binary16 codes (uint16) -> float64: 1 sign, 5 exponent
    (bias 15), 10 mantissa bits."""
    return _decode_binary(bits, 5, 10, 15, fn_nan=False)


def decode_bf16(bits):
    """bfloat16 codes (uint16) -> float64: the upper half of an IEEE-754
    binary32, i.e. 1 sign, 8 exponent (bias 127), 7 mantissa bits."""
    return _decode_binary(bits, 8, 7, 127, fn_nan=False)


def decode_e4m3(bits):
    """OCP FP8 E4M3 "fn" codes (uint8) -> float64: 1 sign, 4 exponent
    (bias 7), 3 mantissa bits, no infinities, NaN only at S.1111.111."""
    return _decode_binary(bits, 4, 3, 7, fn_nan=True)


# ---------------------------------------------------------------------------
# The forward pass
# ---------------------------------------------------------------------------

def causal_allowed(rows, Nq, Nk):
    """Boolean [len(rows), Nk]: key j is visible to query row i iff
    j <= i + (Nk - Nq) (bottom-right aligned causal mask)."""
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.arange(Nk, dtype=np.int64)
    return keys[None, :] <= rows[:, None] + (Nk - Nq)


def _check(q, k, v):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    if q.shape[:2] != k.shape[:2] or k.shape[:3] != v.shape[:3]:
        raise ValueError("batch/head/key dimensions disagree")
    if q.shape[3] != k.shape[3]:
        raise ValueError("q and k head dims differ")
    return q, k, v


def attention(q, k, v, causal, scale, rows=None, row_chunk=1024):
    """Two-pass float64 attention forward.

    q: [B, H, Nq, d]; k: [B, H, Nk, d]; v: [B, H, Nk, dv] (any real dtype,
    widened to float64).  ``scale`` multiplies Q K^T.  ``rows`` optionally
    selects which query rows (absolute indices in 0..Nq-1) to compute; the
    causal mask always uses the absolute index.

    Returns (O [B, H, R, dv] float64, LSE [B, H, R] float64, natural log),
    R = Nq or len(rows).
    """
    q, k, v = _check(q, k, v)
    B, H, Nq, _ = q.shape
    Nk = k.shape[2]
    dv = v.shape[3]
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    scale = float(scale)
    out = np.zeros((B, H, R, dv), dtype=np.float64)
    lse = np.full((B, H, R), -np.inf, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kt = k[b, h].T
            vb = v[b, h]
            for r0 in range(0, R, row_chunk):
                r = rows[r0:r0 + row_chunk]
                # pass 1: scores and their row max over the allowed keys
                s = scale * (q[b, h, r] @ kt)
                if causal:
                    s = np.where(causal_allowed(r, Nq, Nk), s, -np.inf)
                m = s.max(axis=1) if Nk > 0 else np.full(len(r), -np.inf)
                has_key = np.isfinite(m)
                m_ref = np.where(has_key, m, 0.0)
                # pass 2: unnormalised probabilities, their sum, P V, LSE
                p = np.exp(s - m_ref[:, None])
                l = p.sum(axis=1)
                o = p @ vb
                safe_l = np.where(has_key, l, 1.0)
                out[b, h, r0:r0 + len(r)] = np.where(has_key[:, None], o / safe_l[:, None], 0.0)
                lse[b, h, r0:r0 + len(r)] = np.where(has_key, m_ref + np.log(safe_l), -np.inf)
    return out, lse


def attention_blockwise(q, k, v, causal, scale, block):
    """Online-softmax float64 forward, one key block at a time, in the order
    of the consumer loop in the concept card's implementation sketch.

    Same arguments and results as ``attention`` (all rows).  ``block`` is the
    number of keys per step; it need not divide Nk.
    """
    q, k, v = _check(q, k, v)
    B, H, Nq, _ = q.shape
    Nk = k.shape[2]
    dv = v.shape[3]
    block = int(block)
    if block < 1:
        raise ValueError("block must be >= 1")
    scale = float(scale)
    out = np.zeros((B, H, Nq, dv), dtype=np.float64)
    lse = np.full((B, H, Nq), -np.inf, dtype=np.float64)
    all_rows = np.arange(Nq)
    for b in range(B):
        for h in range(H):
            output = np.zeros((Nq, dv))
            row_max = np.full(Nq, -np.inf)
            row_sum = np.zeros(Nq)
            for j0 in range(0, Nk, block):
                j1 = min(Nk, j0 + block)
                scores = scale * (q[b, h] @ k[b, h, j0:j1].T)
                if causal:
                    allowed = causal_allowed(all_rows, Nq, Nk)[:, j0:j1]
                    scores = np.where(allowed, scores, -np.inf)
                new_max = np.maximum(row_max, scores.max(axis=1))
                # a row that has seen no allowed key yet keeps max = -inf;
                # measure its (all zero) probabilities from 0 instead
                ref = np.where(np.isfinite(new_max), new_max, 0.0)
                probs = np.exp(scores - ref[:, None])
                factor = np.exp(row_max - ref)
                row_sum = factor * row_sum + probs.sum(axis=1)
                output = factor[:, None] * output + probs @ v[b, h, j0:j1]
                row_max = new_max
            has_key = row_sum > 0
            safe = np.where(has_key, row_sum, 1.0)
            out[b, h] = np.where(has_key[:, None], output / safe[:, None], 0.0)
            lse[b, h] = np.where(has_key, row_max + np.log(safe), -np.inf)
    return out, lse
