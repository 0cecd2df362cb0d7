"""Float64 CPU oracle for the fused attention forward pass.

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
