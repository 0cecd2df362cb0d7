"""The Python wrappers refuse inputs whose shapes, dtypes or placement the C
ABI cannot see, before any pointer reaches the library (a K with fewer rows
or heads than q says, or a host tensor, would otherwise be read on the
device).  Runs on the CPU: every rejection happens before the library is
called."""

import pytest
import torch

from attention_forward_02_amd import binding as b

F16 = torch.float16


def t(*shape, dtype=F16):
    return torch.zeros(shape, dtype=dtype)


@pytest.mark.parametrize("q,k,v,exc,msg", [
    (t(1, 2, 64, 64), t(1, 2, 64, 64)[0], t(1, 2, 64, 64), ValueError, "4-D"),
    (t(1, 2, 64, 64), t(1, 1, 64, 64), t(1, 1, 64, 64), ValueError, "does not match q"),
    (t(1, 2, 64, 64), t(2, 2, 64, 64), t(2, 2, 64, 64), ValueError, "does not match q"),
    (t(1, 2, 64, 64), t(1, 2, 64, 128), t(1, 2, 64, 128), ValueError, "does not match q"),
    (t(1, 2, 64, 64), t(1, 2, 80, 64), t(1, 2, 64, 64), ValueError, "k's shape"),
    (t(1, 2, 64, 64), t(1, 2, 64, 64), t(1, 2, 64, 64, dtype=torch.bfloat16), TypeError, "one dtype"),
    (t(1, 2, 64, 64), t(1, 2, 64, 64), t(1, 2, 64, 64, dtype=torch.float32), TypeError, "unsupported"),
    (t(1, 2, 64, 64), t(1, 2, 64, 64).transpose(2, 3), t(1, 2, 64, 64), ValueError, "contiguous"),
    (t(1, 2, 64, 64), t(1, 2, 64, 64), t(1, 2, 64, 64), ValueError, "GPU tensor"),
])
def test_attention_rejects(q, k, v, exc, msg):
    with pytest.raises(exc, match=msg):
        b.attention(q, k, v)


def test_quantize_rejects():
    with pytest.raises(ValueError, match="4-D"):
        b.quantize_fp8(t(2, 64, 64))
    with pytest.raises(TypeError, match="float16 or bfloat16"):
        b.quantize_fp8(t(1, 1, 64, 64, dtype=torch.uint8))
    with pytest.raises(ValueError, match="contiguous"):
        b.quantize_fp8(t(1, 1, 64, 64).transpose(2, 3))
    with pytest.raises(ValueError, match="GPU tensor"):
        b.quantize_fp8(t(1, 1, 64, 64))


U8 = torch.uint8
F32 = torch.float32


@pytest.mark.parametrize("qs,ks,vs,exc,msg", [
    (t(1, 2, 1, dtype=F32), t(1, 2, 2, dtype=F32), t(1, 2, 2, dtype=F32), ValueError, r"q_descales must have shape \(1, 2, 2\)"),
    (t(1, 2, 2, dtype=F32), t(1, 1, 2, dtype=F32), t(1, 2, 2, dtype=F32), ValueError, "k_descales must have shape"),
    (t(1, 2, 2, dtype=F32), t(1, 2, 2, dtype=F32), t(1, 2, 3, dtype=F32), ValueError, "v_descales must have shape"),
    (t(1, 2, 2, dtype=F16), t(1, 2, 2, dtype=F32), t(1, 2, 2, dtype=F32), TypeError, "q_descales must be float32"),
    (t(1, 2, 2, dtype=F32), t(1, 2, 2, dtype=F32), t(1, 2, 2, dtype=F32), ValueError, "GPU tensor"),
])
def test_blockscaled_rejects(qs, ks, vs, exc, msg):
    codes = t(1, 2, 100, 64, dtype=U8)
    with pytest.raises(exc, match=msg):
        b.attention_fp8_blockscaled(codes, codes, codes, qs, ks, vs)


def test_blockscaled_rejects_16bit_inputs():
    x = t(1, 2, 100, 64)
    ds = t(1, 2, 2, dtype=F32)
    with pytest.raises(TypeError, match="E4M3"):
        b.attention_fp8_blockscaled(x, x, x, ds, ds, ds)
