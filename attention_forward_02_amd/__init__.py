"""MI355X (gfx950) fused attention forward: a C-ABI HIP library
(libattn.so, declared in include/attn.h) and its thin Python binding.

    from attention_forward_02_amd import attention
    o, lse = attention(q, k, v, causal=True)     # torch device tensors

The library is loaded on first use; nothing here computes on the CPU.
"""

from .binding import (  # noqa: F401
    ATTN_BF16,
    ATTN_ERR_ALIAS,
    ATTN_ERR_ALIGN,
    ATTN_ERR_DTYPE,
    ATTN_ERR_HEADDIM,
    ATTN_ERR_LAUNCH,
    ATTN_ERR_NULL,
    ATTN_ERR_SCALE,
    ATTN_ERR_SHAPE,
    ATTN_ERR_VARIANT,
    ATTN_ERR_WORKSPACE,
    ATTN_F16,
    ATTN_FP8_E4M3,
    ATTN_OK,
    ATTN_VARIANT_AUTO,
    ATTN_VARIANT_PIPELINED,
    ATTN_VARIANT_PINGPONG,
    ATTN_VARIANT_PIPELINED_4STAGE,
    ATTN_VARIANT_PIPELINED_3STAGE,
    ATTN_VARIANT_PRODUCER,
    ATTN_VARIANT_SEQUENTIAL,
    ATTN_VARIANT_SEQUENTIAL_BC32,
    ATTN_VARIANT_SEQUENTIAL_BC128,
    ATTN_VARIANT_SPLIT,
    ATTN_VARIANT_WIDE,
    VARIANT_NAMES,
    AttnError,
    ATTN_FP8_BLOCK_ROWS,
    attention,
    attention_fp8_blockscaled,
    attention_fp8_smoothed,
    attention_splitkv,
    attn_fwd,
    attn_fwd_fp8,
    attn_fwd_fp8_blockscaled,
    attn_fwd_splitkv,
    attn_fwd_splitkv_num_splits,
    attn_fwd_splitkv_workspace_bytes,
    attn_fwd_variant,
    attn_quantize_fp8,
    attn_status_str,
    attn_variant_available,
    load_library,
    quantize_fp8,
    splitkv_workspace,
)
