"""Thin ctypes binding of libattn.so (argument marshalling only).

The C functions keep their names: ``attn_fwd``, ``attn_fwd_fp8``,
``attn_fwd_variant``, ``attn_variant_available``, ``attn_quantize_fp8``,
``attn_fwd_fp8_blockscaled``, ``attn_fwd_splitkv`` (with
``attn_fwd_splitkv_workspace_bytes`` and ``attn_fwd_splitkv_num_splits``)
and ``attn_status_str``
take the same arguments as in include/attn.h, with any pointer given either
as an integer device address or as a torch tensor (its ``data_ptr()``), and
the stream as a torch stream, an integer handle or None (the current torch
stream).  ``attention``, ``attention_splitkv``, ``quantize_fp8``,
``attention_fp8_blockscaled`` and ``attention_fp8_smoothed`` are convenience wrappers that allocate the
outputs with torch and raise ``AttnError`` on a non-zero status.  Every step of the computation runs in the HIP library; if the
library is missing, calls raise instead of falling back to anything else.
"""

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libattn.so")

ATTN_FP8_BLOCK_ROWS = 64

ATTN_F16 = 0
ATTN_BF16 = 1
ATTN_FP8_E4M3 = 2

ATTN_OK = 0
ATTN_ERR_NULL = -1
ATTN_ERR_SHAPE = -2
ATTN_ERR_HEADDIM = -3
ATTN_ERR_DTYPE = -4
ATTN_ERR_ALIGN = -5
ATTN_ERR_SCALE = -6
ATTN_ERR_LAUNCH = -7
ATTN_ERR_ALIAS = -8
ATTN_ERR_VARIANT = -9
ATTN_ERR_WORKSPACE = -10
ATTN_ERR_SCRATCH = -11
ATTN_SPLITKV_SCRATCH_BYTES = 64 << 20

ATTN_VARIANT_AUTO = 0
ATTN_VARIANT_PIPELINED = 1
ATTN_VARIANT_PIPELINED_4STAGE = 2
ATTN_VARIANT_SEQUENTIAL = 3
ATTN_VARIANT_SPLIT = 4
ATTN_VARIANT_PINGPONG = 5
ATTN_VARIANT_PRODUCER = 6
ATTN_VARIANT_WIDE = 7
ATTN_VARIANT_SEQUENTIAL_BC32 = 8
ATTN_VARIANT_SEQUENTIAL_BC128 = 9
ATTN_VARIANT_PIPELINED_3STAGE = 10
VARIANT_NAMES = {ATTN_VARIANT_AUTO: "auto", ATTN_VARIANT_PIPELINED: "pipelined",
                 ATTN_VARIANT_PIPELINED_4STAGE: "pipelined_4stage", ATTN_VARIANT_SEQUENTIAL: "sequential",
                 ATTN_VARIANT_SPLIT: "split", ATTN_VARIANT_PINGPONG: "pingpong",
                 ATTN_VARIANT_PRODUCER: "producer", ATTN_VARIANT_WIDE: "wide",
                 ATTN_VARIANT_SEQUENTIAL_BC32: "sequential_bc32", ATTN_VARIANT_SEQUENTIAL_BC128: "sequential_bc128",
                 ATTN_VARIANT_PIPELINED_3STAGE: "pipelined_3stage"}


class AttnError(RuntimeError):
    def __init__(self, status):
        super().__init__(f"attn status {status}: {attn_status_str(status)}")
        self.status = status


_lib = None


def load_library(path=LIB_PATH):
    """Load libattn.so once and declare its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m attention_forward_02_amd.build`")
    # torch ships a HIP runtime of its own: when torch is present it must be
    # the process's runtime before the library's dependency is resolved, or
    # tensors allocated by one runtime would reach kernels launched by another
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, vp]
    lib.attn_fwd.restype = ci
    lib.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, cf, cf, cf, vp]
    lib.attn_fwd_fp8.restype = ci
    lib.attn_variant_available.argtypes = [ci, ci, ci]
    lib.attn_variant_available.restype = ci
    lib.attn_fwd_variant.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, cf, cf, cf, ci, vp]
    lib.attn_fwd_variant.restype = ci
    lib.attn_quantize_fp8.argtypes = [vp, ci, vp, vp, ci, ci, ci, ci, ci, vp]
    lib.attn_quantize_fp8.restype = ci
    lib.attn_fwd_fp8_blockscaled.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp]
    lib.attn_fwd_fp8_blockscaled.restype = ci
    ull = ctypes.c_ulonglong
    lib.attn_fwd_splitkv_workspace_bytes.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci]
    lib.attn_fwd_splitkv_workspace_bytes.restype = ull
    lib.attn_fwd_splitkv_num_splits.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci]
    lib.attn_fwd_splitkv_num_splits.restype = ci
    lib.attn_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, cf, cf, cf, ci, vp, ull, vp]
    lib.attn_fwd_splitkv.restype = ci
    lib.attn_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, cf, cf, cf, ci, vp]
    lib.attn_fwd_splitkv_noalloc.restype = ci
    lib.attn_status_str.argtypes = [ci]
    lib.attn_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    return int(s)


def attn_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, stream=None):
    """The C ``attn_fwd``; returns its status code."""
    lib = load_library()
    return lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Nq), int(Nk),
                        int(d), int(bool(causal)), float(scale), int(dtype), _stream(stream))


def attn_fwd_fp8(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, q_descale, k_descale, v_descale,
                 stream=None):
    """The C ``attn_fwd_fp8``; returns its status code."""
    lib = load_library()
    return lib.attn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Nq), int(Nk),
                            int(d), int(bool(causal)), float(scale), float(q_descale), float(k_descale),
                            float(v_descale), _stream(stream))


def attn_variant_available(d, dtype, variant):
    """The C ``attn_variant_available``: True if the variant is built for (d, dtype)."""
    return bool(load_library().attn_variant_available(int(d), int(dtype), int(variant)))


def attn_fwd_variant(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, q_descale, k_descale, v_descale,
                     variant, stream=None):
    """The C ``attn_fwd_variant``; returns its status code."""
    lib = load_library()
    return lib.attn_fwd_variant(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Nq), int(Nk),
                                int(d), int(bool(causal)), float(scale), int(dtype), float(q_descale),
                                float(k_descale), float(v_descale), int(variant), _stream(stream))


def attn_quantize_fp8(x, dtype, codes, descales, B, H, N, d, hadamard, stream=None):
    """The C ``attn_quantize_fp8``; returns its status code."""
    lib = load_library()
    return lib.attn_quantize_fp8(_ptr(x), int(dtype), _ptr(codes), _ptr(descales), int(B), int(H), int(N), int(d),
                                 int(bool(hadamard)), _stream(stream))


def attn_fwd_fp8_blockscaled(q, k, v, q_descales, k_descales, v_descales, o, lse, B, H, Nq, Nk, d, causal, scale,
                             stream=None):
    """The C ``attn_fwd_fp8_blockscaled``; returns its status code."""
    lib = load_library()
    return lib.attn_fwd_fp8_blockscaled(_ptr(q), _ptr(k), _ptr(v), _ptr(q_descales), _ptr(k_descales),
                                        _ptr(v_descales), _ptr(o), _ptr(lse), int(B), int(H), int(Nq), int(Nk),
                                        int(d), int(bool(causal)), float(scale), _stream(stream))


def attn_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, causal, dtype, num_splits=0):
    """The C ``attn_fwd_splitkv_workspace_bytes`` (0 for an unsupported d or dtype)."""
    return int(load_library().attn_fwd_splitkv_workspace_bytes(int(B), int(H), int(Nq), int(Nk), int(d),
                                                               int(bool(causal)), int(dtype), int(num_splits)))


def attn_fwd_splitkv_num_splits(B, H, Nq, Nk, d, causal, dtype, num_splits=0):
    """The C ``attn_fwd_splitkv_num_splits``."""
    return int(load_library().attn_fwd_splitkv_num_splits(int(B), int(H), int(Nq), int(Nk), int(d),
                                                          int(bool(causal)), int(dtype), int(num_splits)))


def attn_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, q_descale, k_descale, v_descale,
                     num_splits, workspace, workspace_bytes, stream=None):
    """The C ``attn_fwd_splitkv``; returns its status code."""
    lib = load_library()
    return lib.attn_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Nq), int(Nk),
                                int(d), int(bool(causal)), float(scale), int(dtype), float(q_descale),
                                float(k_descale), float(v_descale), int(num_splits), _ptr(workspace),
                                int(workspace_bytes), _stream(stream))


def attn_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, q_descale, k_descale,
                             v_descale, num_splits, stream=None):
    """The C ``attn_fwd_splitkv_noalloc``; returns its status code."""
    lib = load_library()
    return lib.attn_fwd_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Nq),
                                        int(Nk), int(d), int(bool(causal)), float(scale), int(dtype),
                                        float(q_descale), float(k_descale), float(v_descale), int(num_splits),
                                        _stream(stream))


def attn_status_str(status):
    return load_library().attn_status_str(int(status)).decode()


def _dtype_code(t):
    import torch
    if t.dtype == torch.float16:
        return ATTN_F16
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype in (torch.uint8, getattr(torch, "float8_e4m3fn", None)):
        return ATTN_FP8_E4M3
    raise TypeError(f"unsupported input dtype {t.dtype}")


def _check_device(tensors, names):
    """Every tensor on one GPU: the library dereferences raw device pointers,
    so a host tensor or a second device must be refused here."""
    dev = None
    for t, n in zip(tensors, names):
        if not getattr(t, "is_cuda", False):
            raise ValueError(f"{n} must be a GPU tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{n} is on {t.device}, expected {dev}")


def _check_qkv(q, k, v, placement=True):
    """Shapes, dtypes and placement of q [B,H,Nq,d], k and v [B,H,Nk,d]:
    the C ABI sees only pointers and sizes, so a K or V smaller than the sizes
    taken from q would be read past its end on the device."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t.dim() != 4:
            raise ValueError(f"{n} must be 4-D [B, H, N, d], got shape {tuple(t.shape)}")
    if tuple(k.shape[:2]) != tuple(q.shape[:2]) or k.shape[3] != q.shape[3]:
        raise ValueError(f"k {tuple(k.shape)} does not match q {tuple(q.shape)} in B, H or d")
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"v {tuple(v.shape)} must have k's shape {tuple(k.shape)}")
    code = _dtype_code(q)
    if _dtype_code(k) != code or _dtype_code(v) != code:
        raise TypeError("q, k, v must share one dtype")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if placement:
        _check_device((q, k, v), ("q", "k", "v"))


def _check_descales(ds, name, B, H, N):
    import torch
    nb = (N + ATTN_FP8_BLOCK_ROWS - 1) // ATTN_FP8_BLOCK_ROWS
    if tuple(ds.shape) != (B, H, nb):
        raise ValueError(f"{name} must have shape {(B, H, nb)}, got {tuple(ds.shape)}")
    if ds.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    if not ds.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def attention(q, k, v, causal=False, scale=None, descale=None, stream=None, variant=None):
    """O, LSE for contiguous device tensors q [B,H,Nq,d], k, v [B,H,Nk,d].

    fp16 -> fp16 O, bf16 -> bf16 O, e4m3 (float8_e4m3fn or uint8 codes) ->
    fp16 O with ``descale = (q_descale, k_descale, v_descale)``.  LSE is
    float32 [B,H,Nq].  Runs on ``stream`` (default: current torch stream)
    without synchronising.  ``variant`` (an ATTN_VARIANT_* code) picks a
    kernel variant through ``attn_fwd_variant``; None runs the default.
    """
    import torch
    _check_qkv(q, k, v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out_dtype = torch.bfloat16 if code == ATTN_BF16 else torch.float16
    o = torch.empty((B, H, Nq, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if variant is not None:
        qd, kd, vd = descale if (descale is not None and code == ATTN_FP8_E4M3) else (1.0, 1.0, 1.0)
        st = attn_fwd_variant(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, code, qd, kd, vd, variant, stream)
    elif code == ATTN_FP8_E4M3:
        qd, kd, vd = descale if descale is not None else (1.0, 1.0, 1.0)
        st = attn_fwd_fp8(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, qd, kd, vd, stream)
    else:
        st = attn_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, code, stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return o, lse


def splitkv_workspace(q, k, num_splits=0, causal=False):
    """A device workspace (uint8 tensor, possibly empty) for
    ``attention_splitkv`` on inputs shaped like q and k with the same
    num_splits and causal flag, reusable by later calls on the same
    stream."""
    import torch
    B, H, Nq, d = q.shape
    if attn_fwd_splitkv_num_splits(B, H, Nq, k.shape[2], d, causal, _dtype_code(q), num_splits) == 0:
        raise ValueError("unsupported head dim or dtype")
    n = attn_fwd_splitkv_workspace_bytes(B, H, Nq, k.shape[2], d, causal, _dtype_code(q), num_splits)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)


def attention_splitkv(q, k, v, causal=False, scale=None, descale=None, num_splits=0, workspace=None, stream=None):
    """``attention`` through ``attn_fwd_splitkv``: the key range of every
    query tile split over up to ``num_splits`` workgroups (0 = the library's
    choice, which depends on ``causal``) and merged.  ``workspace`` is a
    device tensor from ``splitkv_workspace`` made with the same num_splits
    and causal flag (allocated here when None); one too small for the call
    raises AttnError (ATTN_ERR_WORKSPACE) before anything runs."""
    import torch
    _check_qkv(q, k, v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = splitkv_workspace(q, k, num_splits, causal)
    elif not getattr(workspace, "is_cuda", False) or workspace.device != q.device:
        raise ValueError("workspace must be a tensor on q's device")
    out_dtype = torch.bfloat16 if code == ATTN_BF16 else torch.float16
    o = torch.empty((B, H, Nq, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    qd, kd, vd = descale if (descale is not None and code == ATTN_FP8_E4M3) else (1.0, 1.0, 1.0)
    nbytes = workspace.numel() * workspace.element_size()
    st = attn_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, code, qd, kd, vd, num_splits, workspace,
                          nbytes, stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return o, lse


def quantize_fp8(x, hadamard=False, stream=None):
    """Block-scaled E4M3 codes of a contiguous fp16/bf16 device tensor x
    [B,H,N,d]: returns (codes uint8 [B,H,N,d], descales float32
    [B,H,ceil(N/64)]), optionally after the 16x16 Walsh-Hadamard transform
    (for Q and K only)."""
    import torch
    if x.dim() != 4:
        raise ValueError(f"x must be 4-D [B, H, N, d], got shape {tuple(x.shape)}")
    code = _dtype_code(x)
    if code == ATTN_FP8_E4M3:
        raise TypeError("x must be float16 or bfloat16")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    _check_device((x,), ("x",))
    B, H, N, d = x.shape
    nb = (N + ATTN_FP8_BLOCK_ROWS - 1) // ATTN_FP8_BLOCK_ROWS
    codes = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
    descales = torch.empty((B, H, nb), dtype=torch.float32, device=x.device)
    st = attn_quantize_fp8(x, code, codes, descales, B, H, N, d, hadamard, stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return codes, descales


def attention_fp8_blockscaled(q, k, v, q_descales, k_descales, v_descales, causal=False, scale=None, stream=None):
    """O (fp16), LSE for block-scaled E4M3 codes (uint8 or float8_e4m3fn
    device tensors [B,H,N,d]) and their float32 descales [B,H,ceil(N/64)]."""
    import torch
    _check_qkv(q, k, v, placement=False)
    if _dtype_code(q) != ATTN_FP8_E4M3:
        raise TypeError("q, k, v must be E4M3 codes (uint8 or float8_e4m3fn)")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _check_descales(q_descales, "q_descales", B, H, Nq)
    _check_descales(k_descales, "k_descales", B, H, Nk)
    _check_descales(v_descales, "v_descales", B, H, Nk)
    _check_device((q, k, v, q_descales, k_descales, v_descales),
                  ("q", "k", "v", "q_descales", "k_descales", "v_descales"))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty((B, H, Nq, d), dtype=torch.float16, device=q.device)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    st = attn_fwd_fp8_blockscaled(q, k, v, q_descales, k_descales, v_descales, o, lse, B, H, Nq, Nk, d, causal,
                                  scale, stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return o, lse


def attention_fp8_smoothed(q, k, v, causal=False, scale=None, stream=None):
    """FP8 attention of fp16/bf16 device tensors through block-scaled E4M3:
    Q and K are quantised after the Walsh-Hadamard transform, V without it,
    then the block-scaled forward runs.  Returns (O fp16, LSE)."""
    q8, qd = quantize_fp8(q, True, stream)
    k8, kd = quantize_fp8(k, True, stream)
    v8, vd = quantize_fp8(v, False, stream)
    return attention_fp8_blockscaled(q8, k8, v8, qd, kd, vd, causal, scale, stream)
