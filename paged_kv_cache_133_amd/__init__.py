"""MI355X-native paged KV cache: slot_mapping write and block-table attention decode.

The compute lives in the HIP library libpagedkv.so (built by
paged_kv_cache_133_amd.build); this package only marshals torch tensors to its C ABI.
"""
