"""JoLT compressed-cache decode attention on MI355X (gfx950).

Python face of libjolt (C ABI in include/jolt.h): load a JoLT-compressed KV
cache to the device and run decode attention directly over its stored factors
and packed residuals, plus a dense decode comparator.  See ``_jolt`` for the
functions; they keep the C names.
"""
from ._jolt import (  # noqa: F401
    Cache, JoltError, KERNEL_AUTO, KERNEL_GENERIC, KERNEL_MFMA, LIB_PATH, EXPORTS,
    jolt_load_cache, jolt_decode_workspace_size, jolt_decode_attention,
    jolt_decode_tail_workspace_size, jolt_decode_attention_tail,
    jolt_dense_workspace_size, jolt_dense_attention, jolt_make_rotation, jolt_debug_unpack, jolt_debug_sincos,
    jolt_last_error, lib, jolt_flash_spectra, jolt_flash_compress_cell, jolt_quantize_rows,
    jolt_decode_attention_noalloc, jolt_noalloc_scratch_bytes, jolt_allocate,
    jolt_flash_layer_groups,
)
