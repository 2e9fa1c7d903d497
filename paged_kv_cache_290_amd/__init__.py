"""Paged-KV attention for MI355X (gfx950): a C-ABI HIP library plus a thin binding.

    from paged_kv_cache_290_amd import kv_write, attention, workspace_size

The shared library is loaded lazily on the first call and must have been built with
`python -m paged_kv_cache_290_amd.build`.
"""
from .ops import (BLOCK_SIZE, BlockAllocator, StepBatch, attention,  # noqa: F401
                  attention_shared_prefix, attention_with_write,
                  attention_with_write_noalloc, block_keys, shared_prefix_workspace_size,
                  validate_shared_prefix, copy_blocks, kv_write, plan_step,
                  read_probe, swap_bytes, swap_in, swap_out, validate_metadata, workspace_size)
from ._lib import PagedKVError  # noqa: F401
