"""PagedAttention decode, paged KV write, block copy and multi-token attention
for AMD MI355X (gfx950).

The compute lives in libpagedkv.so (hand-written HIP kernels behind a C ABI,
declared in include/pagedkv.h); this package is its thin Python binding plus
host-side block bookkeeping.  There is no fallback: if the library is not
built, every call raises.
"""

from ._lib import (
    ContractError,
    PKV_BF16,
    PKV_F32,
    PKV_FP8_E4M3,
    PagedKVError,
    decode_partition_size,
    decode_workspace_size,
    decode_workspace_counter_bytes,
    dtype_code,
    hbm_gather_probe,
    hbm_read_probe,
    load,
    decode_noalloc_max_workspace,
    paged_attention_decode,
    paged_attention_decode_noalloc,
    paged_attention_decode_partitions,
    paged_attention_decode_reduce,
    paged_attention_decode_shared_prefix,
    paged_attention_decode_write,
    paged_attention_prefill,
    paged_kv_block_copy,
    prefill_workspace_size,
    paged_kv_cache_write,
    shared_prefix_workspace_size,
    status_string,
    write_workspace_size,
)
from .block_manager import BlockManager, OutOfBlocks

__all__ = [
    "ContractError", "PKV_BF16", "PKV_F32", "PKV_FP8_E4M3", "PagedKVError", "BlockManager", "OutOfBlocks",
    "decode_partition_size", "decode_workspace_size", "decode_workspace_counter_bytes", "dtype_code", "hbm_gather_probe",
    "hbm_read_probe", "load",
    "decode_noalloc_max_workspace", "paged_attention_decode",
    "paged_attention_decode_noalloc", "paged_attention_decode_partitions",
    "paged_attention_decode_reduce", "paged_attention_decode_shared_prefix",
    "paged_attention_decode_write",
    "paged_attention_prefill", "paged_kv_block_copy", "paged_kv_cache_write",
    "prefill_workspace_size", "shared_prefix_workspace_size",
    "status_string",
    "write_workspace_size",
]
