"""pkv: paged KV-cache decode attention and cache maintenance on MI355X (gfx950).

A thin ctypes binding over ``libpkv.so`` (C ABI declared in ``include/pkv.h``
and, for the host block manager, ``include/pkv_block_manager.h``).
Every operation runs in the library's HIP kernels; this module only checks
tensor shapes, dtypes and devices and marshals pointers, sizes and the
current HIP stream.  There is no fallback: if the library is missing or the
tensors are not on the GPU, calls raise.
"""
from ._binding import (  # noqa: F401
    PKVError,
    PKV_F32, PKV_F16, PKV_BF16,
    PKV_SWAP_IN, PKV_SWAP_OUT,
    EXPORTED_SYMBOLS,
    library,
    library_path,
    paged_attention_decode,
    paged_attention_decode_noalloc,
    noalloc_scratch_bytes,
    paged_attention_decode_shared,
    paged_attention_partitions_planned_shared,
    paged_attention_partitions_planned_fp8,
    paged_attention_decode_fp8,
    paged_attention_decode_int8,
    paged_attention_prefill,
    paged_attention_prefill_workspace_size,
    reshape_and_cache_fp8,
    reshape_and_cache_int8,
    paged_attention_partitions,
    paged_attention_partitions_planned,
    paged_attention_plan,
    paged_attention_plan_and_cache,
    paged_attention_plan_and_cache_fp8,
    paged_attention_plan_and_cache_shared,
    paged_attention_plan_fp8,
    paged_attention_plan_shared,
    paged_attention_reduce,
    paged_attention_workspace_size,
    reshape_and_cache,
    copy_blocks,
    swap_blocks,
    decode_bytes,
    stream_read,
)
from .block_manager import BlockManager  # noqa: F401
