"""Sliding-window attention with a learnable sink on MI355X (gfx950).

A thin Python binding over the C ABI of libhswa.so (include/hswa.h).  It
only marshals arguments: torch supplies device memory and the current HIP
stream, and every step of the computation runs in the library's kernels.
There is no fallback: if the library is missing, load() raises.
"""

from ._binding import (  # noqa: F401
    EXPORTED_SYMBOLS,
    HswaError,
    KV_CONTIGUOUS,
    KV_RING,
    NOALLOC_SCRATCH_BYTES,
    decode_multi_workspace_size,
    decode_workspace_size,
    ga_prefill,
    gather_probe,
    kv_cache_append,
    lib_path,
    load,
    prefill_workspace_size,
    sparse_sink_attn,
    sparse_select_tokens,
    sparse_sink_attn_fp8,
    sparse_workspace_size,
    stream_probe,
    swa_sink_decode,
    swa_sink_decode_multi,
    swa_sink_decode_noalloc,
    swa_sink_decode_fp8,
    swa_sink_prefill,
    swa_sink_prefill_chunk,
    swa_sink_prefill_chunk_cached,
    version,
)
