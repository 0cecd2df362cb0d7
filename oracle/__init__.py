"""Float64 CPU oracle for the fused attention forward pass and for the
block-scaled, Hadamard-smoothed FP8 quantisation of its inputs.

Test infrastructure: only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import it.  The product library never does.
"""

from .forward import (  # noqa: F401
    attention,
    attention_blockwise,
    causal_allowed,
    decode_bf16,
    decode_e4m3,
    decode_f16,
)
from .fp8_block import (  # noqa: F401
    BLOCK_ROWS,
    dequantize_blocks,
    encode_e4m3,
    hadamard16,
    hadamard_matrix,
    quantize_blocks,
)
