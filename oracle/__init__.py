"""CPU oracle for sliding-window attention with a learnable sink and its siblings.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, calls or links this package.  Only the test
suite, the smoke check and the CPU-baseline leg of the benchmark may use it.

What it computes is the plain definition from the pages, in float64 with a
two-pass direct summation (max first, then exponentials and sums):

  * "MiMo-V2-Flash: Hybrid Sliding Window Attention Architecture" (rslog.cc):
    section 1.2 (scaled scores), 2.1 (causal window), 4.2 (sink in the
    denominator), 4.4 (max-stabilised form and output), 5 (GA layers carry
    no sink term).
  * "39 SWA + 9 GA layers: MiMo-V2.6-Flash hybrid SWA" (pwwt.cn): tables in
    sections 3 and 4 (heads, head dims), section 5 (two RoPE bases, partial
    rotary factor).
  * "MiMo-V3 HySparse2" (aideepthink.cn), section 4: forced-recent window of
    128 tokens plus up to 1024 selected tokens in one sparse attention.
  * "MiMo v2.5 inference optimisation" (youngju.dev), KV-cache restructuring
    and scheduling: the dual-pool KV cache (the SWA pool holds W slots, the
    full-attention pool holds the sequence) and prefill in fixed-size chunks
    behind a cached prefix; the closing section's FP8 cache (with
    aideepthink.cn section 5), read as OCP E4M3 codes with one scale per kv
    head.

Every function is pinned by tests in tests/test_oracle_pins.py against
closed forms, library routines and brute force.  The RoPE pairing
convention is a reading (the pages give only the fraction and the bases);
its implementation is pinned by closed forms, the choice itself is
"parity unpinned".
"""

from .attention import (  # noqa: F401
    rotary_dims,
    rope,
    window_keys,
    ring_slot_positions,
    sparse_keys,
    attend_row,
    swa_sink_prefill,
    swa_sink_prefill_chunk,
    swa_sink_prefill_chunk_cached,
    ga_prefill,
    swa_sink_decode_ring,
    swa_sink_decode_contiguous,
    decode_multi_ring,
    decode_multi_contiguous,
    e4m3_value,
    dequantise_kv,
    e4m3_encode,
    rope_f32_steps,
    kv_append,
    swa_sink_decode_ring_fp8,
    swa_sink_decode_contiguous_fp8,
    sparse_sink_attn,
    prefill_rows,
    sparse_rows,
    sparse_rows_fp8,
    selection_importance,
    select_tokens,
)
