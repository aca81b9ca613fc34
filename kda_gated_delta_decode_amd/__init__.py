"""MI355X-native KDA (Kimi Delta Attention) recurrent decode.

The decode update runs in hand-written gfx950 HIP kernels behind a C ABI
(include/kda_decode.h, built into libkda_decode.so by
``python -m kda_gated_delta_decode_amd.build``).  This package is the thin
Python binding: ``binding.kda_decode_step`` and the other entry points carry
the C names and only marshal arguments.
"""
from .binding import (  # noqa: F401
    KDA_BF16, KDA_F16, KDA_F32, KDA_MAX_ROWS, KdaError, kda_abi_version, kda_copy_probe,
    kda_decode_step, kda_decode_step_conv, kda_describe_launch, kda_pool_bytes, kda_prefill,
    kda_prefill_validate, kda_state_at, kda_state_copy, kda_strerror, kda_tile_bv, kda_tile_of_block, kda_validate, library, make_conv_pool, make_pool,
)
