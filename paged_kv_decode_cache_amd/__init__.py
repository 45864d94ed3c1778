"""Paged KV-cache decode attention for AMD Instinct MI355X (gfx950).

The computation lives in libpkv.so (hand-written HIP kernels behind a C ABI,
``include/pkv.h``); this package is its thin Python binding.
"""
from ._binding import (LIB_PATH, HEADER_PATH, load_library, declared_functions,
                       status_string, LaunchConfig, kv_cache_append,
                       paged_attention_decode, paged_attention_decode_split,
                       split_reduce, max_partitions_for, paged_decode_step, StepWorkspace,
                       paged_decode_step_noalloc, PKV_ERR_SCRATCH,
                       paged_attention_prefill, paged_attention_prefill_split,
                       kv_cache_append_q8, paged_attention_decode_q8,
                       paged_attention_decode_split_q8, paged_decode_step_q8,
                       BlockAllocator, NoSpaceError, PKV_ERR_NO_SPACE,
                       PKV_OK, PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_LAUNCH)

__all__ = ["LIB_PATH", "HEADER_PATH", "load_library", "declared_functions", "status_string",
           "LaunchConfig", "kv_cache_append", "paged_attention_decode",
           "paged_attention_decode_split", "split_reduce", "max_partitions_for",
           "paged_decode_step", "StepWorkspace", "paged_decode_step_noalloc", "PKV_ERR_SCRATCH",
           "paged_attention_prefill",
           "paged_attention_prefill_split",
           "kv_cache_append_q8", "paged_attention_decode_q8", "paged_attention_decode_split_q8",
           "paged_decode_step_q8",
           "BlockAllocator", "NoSpaceError", "PKV_ERR_NO_SPACE",
           "PKV_OK", "PKV_ERR_INVALID_ARG", "PKV_ERR_UNSUPPORTED", "PKV_ERR_LAUNCH"]
