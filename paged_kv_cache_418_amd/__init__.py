"""Paged-KV attention for AMD MI355X (gfx950).

The compute path is the HIP library libpa.so (C ABI in include/pa.h); the
functions re-exported here are its ctypes binding and take GPU torch tensors.
``workloads`` holds the seeded synthetic inputs.
"""
from ._binding import (  # noqa: F401
    BlockPool, pool_hash_blocks, PA_BF16, PA_F32, PA_FP8_E4M3, PAError, abi_version, header_symbols, load,
    pa_decode, pa_decode_cascade, pa_decode_cascade_fp8, pa_decode_cascade_workspace_bytes, pa_decode_cascade_write,
    pa_decode_cascade_write_fp8, pa_decode_fp8,
    pa_decode_local, pa_decode_local_fp8, pa_decode_local_write, pa_decode_local_write_fp8, pa_decode_static,
    pa_decode_window, pa_decode_window_fp8, pa_decode_window_write, pa_decode_window_write_fp8, pa_decode_write,
    pa_decode_write_fp8,
    pa_decode_workspace_bytes, pa_prefill_varlen, pa_prefill_varlen_fp8, pa_prefill_varlen_fp8_workspace_bytes,
    pa_prefill_varlen_write,
    pa_prefill_varlen_local, pa_prefill_varlen_local_fp8, pa_prefill_varlen_local_workspace_bytes,
    pa_prefill_varlen_window, pa_prefill_varlen_window_fp8, pa_prefill_varlen_window_workspace_bytes,
    pa_prefill_varlen_workspace_bytes, pa_reshape_and_cache, pa_reshape_and_cache_fp8, pa_slot_mapping, pa_write_kv,
    set_fused, set_validate, timing_enable, timing_read, timing_reset)
