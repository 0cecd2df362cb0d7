"""Float64 CPU oracle for block-scaled FP8 E4M3 quantisation with incoherent
(Walsh-Hadamard) processing of Q and K.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the
``cpu_baseline`` leg of the benchmark use it.  It shares no code with the
HIP library and imports nothing but NumPy and the decoders of
``oracle.forward``.

What it computes ("Inside FlashAttention-3 & Warp-Specialized CUDA Kernels",
section 5, the second item, block scaling with Hadamard outlier smoothing):

* ``hadamard16`` multiplies the last axis by a block-diagonal orthogonal
  matrix made of d/16 copies of the 16x16 Walsh-Hadamard matrix divided by 4
  (Sylvester's construction: H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]).
  Because that matrix times its transpose is the identity, transforming both
  Q and K leaves every score Q K^T unchanged, while a large entry of one
  channel is spread over the 16 channels of its block.
* ``quantize_blocks`` rounds (optionally transformed) values to E4M3 codes
  with one float32 descale per block of rows.
* ``dequantize_blocks`` gives the real values the codes stand for.
* ``encode_e4m3`` is the OCP FP8 E4M3 ("fn") encoder from the format
  definition: round to nearest, ties to the even code, saturate at 448.

Readings where the page is silent (each is listed in the design notes):

* the transform is applied to Q and K only (the two tensors the page names);
  V is block-quantised without it;
* a block is 64 consecutive rows of one (batch, head) across all d columns,
  the last block of a head holding the remaining rows;
* the transform is exact (float64; exact for binary16 inputs) and its
  result is rounded to float32 once; quantisation works on those float32
  values: descale = fp32(amax / 448) and code = RNE-saturate(fp32(y /
  descale)), both divisions in IEEE float32; a block whose amax is 0 gets
  descale 1 (all codes 0).

Parity status: every function is pinned by the CPU tests (the closed form
of the Walsh-Hadamard entries, the dot-product identity, exhaustive codec
round trips and midpoints, an independent encoder, block independence and
error bounds); none is "parity unpinned".
"""

import numpy as np

from .forward import decode_e4m3

__all__ = [
    "BLOCK_ROWS",
    "E4M3_MAX",
    "hadamard_matrix",
    "hadamard16",
    "encode_e4m3",
    "quantize_blocks",
    "dequantize_blocks",
]

BLOCK_ROWS = 64
E4M3_MAX = 448.0


def hadamard_matrix(n):
    """n x n Walsh-Hadamard matrix of +-1 entries (Sylvester's doubling)."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    if h.shape[0] != n:
        raise ValueError("n must be a power of two")
    return h


_H16 = hadamard_matrix(16) / 4.0  # orthogonal: _H16 @ _H16.T == I


def hadamard16(x):
    """x times the block-diagonal orthogonal Walsh-Hadamard matrix along the
    last axis (d, a multiple of 16), in float64."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 16:
        raise ValueError("last dimension must be a multiple of 16")
    blocks = x.reshape(x.shape[:-1] + (d // 16, 16))
    return (blocks @ _H16.T).reshape(x.shape)


def encode_e4m3(y):
    """E4M3 "fn" codes (uint8) of real values: round to nearest with ties to
    the even code, magnitudes past the largest finite value 448 saturate to
    it.  Normal values are (1 + m/8) 2^(e-7) for e = 1..15 (m = 7 only below
    e = 15); subnormals are m/8 * 2^-6.  Inputs must be finite."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    # binade of a (its exponent), no lower than the subnormal binade's -6;
    # the code grid there has spacing 2^(binade - 3)
    _, ex = np.frexp(a)
    binade = np.maximum(ex - 1, -6)
    spacing = np.ldexp(1.0, binade - 3)
    value = np.rint(a / spacing) * spacing  # rint: ties to even
    value = np.minimum(value, E4M3_MAX)
    _, vex = np.frexp(value)
    sub = value < 2.0 ** -6
    e_field = np.where(sub, 0, vex - 1 + 7)
    m_field = np.where(sub, value / 2.0 ** -9, value / np.ldexp(1.0, vex - 1) * 8 - 8)
    code = (e_field.astype(np.int64) << 3) | np.rint(m_field).astype(np.int64)
    code = np.where(np.signbit(y), code | 0x80, code)
    return code.astype(np.uint8)


def quantize_blocks(x, hadamard, block_rows=BLOCK_ROWS):
    """Block-scaled E4M3 quantisation of x [B, H, N, d] (real values, e.g.
    decoded binary16 / bfloat16 inputs).

    With ``hadamard`` the values are first transformed by ``hadamard16``.
    Returns (codes uint8 [B, H, N, d], descales float32 [B, H, nb]) with
    nb = ceil(N / block_rows); block b covers rows b*block_rows .. +block_rows-1.
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 4:
        raise ValueError("x must be [B, H, N, d]")
    B, H, N, d = x.shape
    y32 = (hadamard16(x) if hadamard else x).astype(np.float32)
    nb = -(-N // block_rows)
    codes = np.empty((B, H, N, d), dtype=np.uint8)
    descales = np.empty((B, H, nb), dtype=np.float32)
    for blk in range(nb):
        r0, r1 = blk * block_rows, min(N, (blk + 1) * block_rows)
        yb = y32[:, :, r0:r1, :]
        amax = np.abs(yb).max(axis=(2, 3))
        ds = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        q = (yb / ds[:, :, None, None]).astype(np.float32)
        codes[:, :, r0:r1, :] = encode_e4m3(q)
        descales[:, :, blk] = ds
    return codes, descales


def dequantize_blocks(codes, descales, block_rows=BLOCK_ROWS):
    """Real values (float64 [B, H, N, d]) of block-scaled E4M3 codes."""
    vals = decode_e4m3(codes)
    N = vals.shape[2]
    rows = np.arange(N) // block_rows
    return vals * np.asarray(descales, dtype=np.float64)[:, :, rows, None]
