"""CPU fp64 oracle for decode attention over a grouped-query KV cache.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library under
``decode_attention_kv_02_amd`` never does, and the two share no code.

The arithmetic lives in ``attn_decode_oracle.c`` (plain C, IEEE double, built
with gcc without fast-math or FP contraction).  This module only compiles it
and marshals numpy arrays through ctypes.
"""
from .oracle import (  # noqa: F401
    build_oracle,
    float_to_half_bits,
    half_to_double,
    oracle_attn_decode,
    oracle_attn_decode_cache,
    oracle_attn_decode_cache_cb,
    oracle_attn_decode_cb,
    oracle_codebook_encode,
    oracle_fwht_undo,
    oracle_kv_append,
    oracle_kv_append_cb,
    oracle_library_path,
    quantize_blocks,
)
