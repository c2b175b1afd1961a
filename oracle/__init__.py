"""CPU oracle for the Q4_0 weight-only linear layer (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package.  It shares no code with the HIP library or its binding.
"""

from .q4_0_oracle import (  # noqa: F401
    BLOCK_BYTES,
    QK,
    bf16_bits_to_f64,
    dequantize,
    embed,
    error_bound,
    gguf_bytes,
    gguf_decode,
    gguf_encode,
    linear,
    linear_rows,
    linear_with_bound,
    pack,
    packed_bytes,
    padded_dims,
    quantize,
    Q41_BLOCK_BYTES,
    q41_decode,
    q41_dequantize,
    q41_encode,
    q41_linear_with_bound,
    q41_pack,
    q41_packed_bytes,
    q41_quantize,
    silu,
    swiglu,
    swiglu_bound,
    swiglu_rows,
)
