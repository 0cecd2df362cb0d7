"""Helpers shared by the GPU tests: upload the generator's bits, run the HIP
path through the C ABI, decode with the oracle's decoders, and compare
against the oracle with the stated tolerances.

Tolerances (written here, used by every GPU parity test):
* fp16 / bf16 inputs: |O_gpu - O_ref| <= 4e-3 + 0.5 * ulp_out(max(|O_ref|, |O_gpu|))
  per element, and |LSE_gpu - LSE_ref| <= 1e-3.  The half-ulp term is the
  rounding of the exact result to the output format; it is below 1e-3 for
  fp16 outputs of magnitude < 4 and only matters for bf16 outputs of
  magnitude >= 1 (early causal rows average few values of V).
* fp8 e4m3 inputs: relative RMSE ||O_gpu - O_ref||_F / ||O_ref||_F <= 3e-2
  over the tensor, O_ref from the oracle on the dequantised inputs.  LSE
  has no stated fp8 gate; the bound used is derived from the arithmetic:
  |LSE_gpu - LSE_ref|_i <= 1e-3 + max_j |dS_ij|, where dS is the score error
  of the E4M3 matrix core.  Its 64-term dot products are not exact in fp32:
  measured over random E4M3 operands (workload-like, uniform over all
  codes, small magnitudes) the error of one 32x32x64 product element stayed
  below 5.1e-4 times the largest |a_k b_k| of that dot product.  With
  FP8_DOT_EPS = 2^-10 (a 2x margin) and d/64 dot products per score,
  max_j |dS_ij| <= FP8_DOT_EPS * scale * (d/64) * max_k |q_ik| max_j |k_jk|,
  and the softmax-weighted LSE error is at most max_j |dS_ij|.
"""

import sys

import numpy as np
import torch

import oracle
from attention_forward_02_amd import attention

O_ATOL = 4e-3
LSE_ATOL = 1e-3
FP8_REL_RMSE = 3e-2
FP8_DOT_EPS = 2.0 ** -10


def fp8_lse_tol(q, k, scale):
    """Per-row LSE tolerance for E4M3 inputs (float64 q [B,H,Nq,d], k
    [B,H,Nk,d], dequantised); see the module docstring."""
    d = q.shape[-1]
    colmax = np.abs(k).max(axis=2, keepdims=True)          # [B,H,1,d]
    m = (np.abs(q) * colmax).max(axis=-1)                  # [B,H,Nq]
    return LSE_ATOL + FP8_DOT_EPS * scale * (d / 64.0) * m


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def upload(bits, dtype):
    if dtype == "e4m3":
        return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.float8_e4m3fn).cuda()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16).cuda()


def decode(bits, dtype):
    if dtype == "f16":
        return oracle.decode_f16(bits)
    if dtype == "bf16":
        return oracle.decode_bf16(bits)
    return oracle.decode_e4m3(bits)


def out_dtype(dtype):
    return "bf16" if dtype == "bf16" else "f16"


def run_gpu(inp, stream=None):
    """Returns (O codes as uint16 numpy, LSE float32 numpy)."""
    q, k, v = upload(inp.q, inp.dtype), upload(inp.k, inp.dtype), upload(inp.v, inp.dtype)
    desc = tuple(float(x) for x in inp.descale) if inp.dtype == "e4m3" else None
    o, lse = attention(q, k, v, causal=inp.causal, scale=float(inp.scale), descale=desc, stream=stream)
    torch.cuda.synchronize()
    return o.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy()


def dequant(inp, heads=None):
    """float64 inputs exactly as the GPU sees them, optionally for a list of
    (b, h) pairs only (returned with B = 1, H = len(heads))."""
    q, k, v = inp.q, inp.k, inp.v
    if heads is not None:
        q = np.stack([q[b, h] for b, h in heads])[None]
        k = np.stack([k[b, h] for b, h in heads])[None]
        v = np.stack([v[b, h] for b, h in heads])[None]
    qd, kd, vd = (float(x) for x in inp.descale)
    return decode(q, inp.dtype) * qd, decode(k, inp.dtype) * kd, decode(v, inp.dtype) * vd


def ulp(x, dtype):
    """Spacing of the output format at |x| (float64 array)."""
    man, emin = (10, -14) if dtype == "f16" else (7, -126)
    a = np.abs(x)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** emin)))
    return np.exp2(e - man)


def compare(o_codes, lse, o_ref, lse_ref, dtype, label="", lse_tol=None):
    """Assert the tolerances above; return a dict of the observed errors.
    `lse_tol` (per row, broadcastable to lse) replaces LSE_ATOL when given."""
    od = out_dtype(dtype)
    o = decode(o_codes, od)
    assert np.isfinite(o).all(), f"{label}: non-finite output"
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin), f"{label}: LSE finiteness differs"
    assert np.all(lse[~fin] == -np.inf), f"{label}: empty rows must have LSE = -inf"
    dl = np.abs(lse[fin].astype(np.float64) - lse_ref[fin]) if fin.any() else np.zeros(1)
    if lse_tol is None:
        ltol = np.full(dl.shape, LSE_ATOL)
    else:
        ltol = np.broadcast_to(lse_tol, lse.shape)[fin] if fin.any() else np.full(1, LSE_ATOL)
    do = np.abs(o - o_ref)
    stats = dict(max_abs_dO=float(do.max()), n_over_4e3=int((do > O_ATOL).sum()), max_abs_dLSE=float(dl.max()))
    if dtype == "e4m3":
        rel = float(np.sqrt(np.sum(do ** 2)) / max(np.sqrt(np.sum(o_ref ** 2)), 1e-300))
        stats["rel_rmse"] = rel
        assert rel <= FP8_REL_RMSE, f"{label}: fp8 relative RMSE {rel:.4g} > {FP8_REL_RMSE}"
    else:
        tol = O_ATOL + 0.5 * ulp(np.maximum(np.abs(o_ref), np.abs(o)), od)
        bad = do > tol
        assert not bad.any(), (f"{label}: {int(bad.sum())} outputs beyond tolerance, worst "
                               f"{float((do - tol).max()):.3g} over; max |dO| {stats['max_abs_dO']:.3g}")
    bad_l = dl > ltol
    assert not bad_l.any(), (f"{label}: {int(bad_l.sum())} LSE beyond tolerance; max |dLSE| {dl.max():.3g}, "
                             f"worst over {float((dl - ltol).max()):.3g}")
    return stats
