"""libdemo: the DeMo / FlexDeMo optimizer step on one parameter shard, as
hand-written HIP kernels for AMD Instinct MI355X (gfx950) behind a C ABI
(include/demo.h).  This package holds the kernels' sources (csrc/), the build
step and the ctypes binding; PyTorch supplies device memory and streams.
"""
from .binding import (  # noqa: F401
    ABI_VERSION,
    CHUNK,
    SCHEME_DCT,
    SCHEME_DILOCO,
    SCHEME_RANDOM,
    SCHEME_STRIDE,
    VAL_F16,
    VAL_F32,
    VAL_TERNARY,
    AdamW,
    Config,
    DemoError,
    demo_abi_version,
    demo_decode_apply,
    demo_decode_apply_adamw,
    demo_encode,
    demo_encode_adamw,
    demo_payload_layout,
    demo_random_select,
    demo_strerror,
)
