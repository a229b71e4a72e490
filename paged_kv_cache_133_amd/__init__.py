"""MI355X-native paged KV cache: slot_mapping write and block-table attention decode.

The compute lives in the HIP library libpagedkv.so (built by
`python -m paged_kv_cache_133_amd.build`); this package only marshals torch tensors
to its C ABI (include/pagedkv.h).  Calls raise if the library is missing.
"""
from ._lib import (BlockManager, CapturedStep, PagedKVError, decode_workspace_size,  # noqa: F401
                   kv_cache_append, kv_cache_copy_blocks, kv_cache_write, kv_cache_write_int8,
                   kv_cache_write_int8_mla, paged_attn_decode_mla_int8,
                   paged_attn_decode_mla_int8_append,
                   kv_rmsnorm_rope_cache, lib, new_decode_workspace, paged_attn_decode,
                   paged_attn_decode_int8, paged_attn_decode_int8_append, paged_attn_decode_append,
                   paged_attn_decode_mla_append,
                   paged_attn_decode_append_noalloc, paged_attn_decode_mtp,
                   paged_attn_decode_mtp_append,
                   paged_attn_varlen, paged_attn_varlen_append,
                   slot_mapping, upload, version)
