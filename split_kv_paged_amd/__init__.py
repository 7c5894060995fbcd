"""split_kv_paged_amd — paged split-KV decode/verify attention for MI355X.

The compute path is libskv.so (HIP kernels for gfx950 behind the C ABI in
include/skv.h); this package only binds it. Build with
`python -m split_kv_paged_amd.build`.
"""
from ._lib import (ATTN_CLAIM_UNITS, CONTRACT_BITS, CONVERT_DIR, EXPORTED, KV_DTYPE, LAYOUT, LIB_PATH,
                   STATIC_SCRATCH_BYTES, SkvError, check_inputs, paged_decode_attn_static,
                   io_dtype, kv_cache_write, kv_page_convert, kv_page_shuffle,
                   kv_page_unshuffle, load, paged_decode_attn, plan_build, plan_words, segment_attn, split_reduce,
                   strerror, workspace_bytes)

__all__ = ["ATTN_CLAIM_UNITS", "CONTRACT_BITS", "CONVERT_DIR", "EXPORTED", "KV_DTYPE", "LAYOUT", "LIB_PATH",
           "STATIC_SCRATCH_BYTES", "SkvError", "check_inputs", "paged_decode_attn_static",
           "io_dtype", "kv_cache_write", "kv_page_convert", "kv_page_shuffle", "kv_page_unshuffle",
           "load", "paged_decode_attn", "plan_build", "plan_words", "segment_attn", "split_reduce",
           "strerror", "workspace_bytes"]
