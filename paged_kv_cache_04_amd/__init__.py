"""paged_kv_cache_04_amd: attention over a paged KV cache on MI355X (gfx950).

The compute lives in libpkv.so (hand-written HIP kernels behind a C ABI,
declared in include/pkv.h).  This package holds the thin Python binding over
that library, the seeded workload generators and the work/byte accounting.
"""
from .binding import (  # noqa: F401
    CacheDesc,
    DecodeOpts,
    PkvError,
    cache_desc,
    decode_opts,
    decode_plan,
    decode_split_for_lens,
    gather_kv,
    kv_append,
    kv_append_quant,
    merge_states,
    noalloc_scratch_bytes,
    paged_attn_decode,
    paged_attn_decode_append,
    paged_attn_decode_append_noalloc,
    paged_attn_decode_append_partials,
    paged_attn_decode_partials,
    paged_attn_decode_shared_prefix,
    paged_attn_mixed,
    paged_attn_prefill_chunk,
    shared_prefix_plan,
    validate_tables,
)
