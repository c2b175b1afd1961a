"""MI355X-native GGUF Q4_0 weight-only linear layer.

The computation lives in libq4amd.so (HIP kernels for gfx950 behind the C ABI
of include/q4_0.h); this package is its thin Python binding.  The library is
loaded on first use and a missing build raises instead of falling back.
"""

from ._binding import (  # noqa: F401
    EXPORTS,
    PackedWeight,
    Q4Error,
    dequant,
    embed,
    embed_gguf,
    gguf_bytes,
    lib,
    library_path,
    linear,
    linear_kernel,
    linear_multi,
    linear_swiglu,
    linear_swiglu_kernel,
    pack,
    packed_bytes,
    quantize,
    PackedWeightQ41,
    q41_dequant,
    q41_linear,
    q41_linear_kernel,
    q41_pack,
    q41_packed_bytes,
    q41_quantize,
    reference_mfma,
    reference_read,
    status_str,
    time_next_launch,
    unpack,
)
