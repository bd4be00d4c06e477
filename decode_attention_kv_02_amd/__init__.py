"""MI355X-native split-KV decode attention over a grouped-query KV cache.

The compute path is the C-ABI library ``libattn_decode.so`` (hand-written HIP
kernels for gfx950) declared in ``include/attn_decode.h``; ``binding`` only
marshals arguments.  Importing the package does not load the library; the
first call does, and raises if it is missing (there is no fallback).
"""
from .binding import (  # noqa: F401
    AttnDecodeError,
    attn_decode,
    attn_decode_cache,
    attn_decode_ex,
    attn_decode_plan,
    attn_decode_release,
    attn_kv_append,
    library_path,
    load_library,
)
