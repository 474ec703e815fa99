"""Paged KV-cache decode attention for AMD MI355X (gfx950).

The work happens in libpkv.so (hand-written HIP kernels behind a C ABI, see
include/pkv.h); this package only loads it and marshals torch tensors.
"""
from ._lib import (HipError, InvalidArg, OutOfBlocks, PkvError, RefcountError,  # noqa: F401
                   Unsupported, WorkspaceError, lib)
from .api import (BLOCK_SIZE, alloc_workspace, copy_blocks, decode_algo_for,  # noqa: F401
                  decode_partition_size, decode_workspace_size, kv_bytes_per_token,
                  multiquery_partition_size, multiquery_workspace_size, paged_cache_append,
                  paged_cache_append_per_channel, paged_decode_attention_per_channel,
                  paged_decode_attention, paged_decode_attention_appending,
                  paged_decode_attention_noalloc,
                  paged_multiquery_attention,
                  stream_read_probe, swap_blocks)
from .pool import BlockPool  # noqa: F401
