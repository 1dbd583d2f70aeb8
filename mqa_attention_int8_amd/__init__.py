"""MI355X-native multi-query attention over an int8 KV cache.

The compute lives in libmqa_int8.so (hand-written HIP for gfx950, C ABI in
include/mqa_int8.h); ``binding`` marshals torch tensors to it.
"""
from .binding import (KVView, MQAError, append_kv, kv_quantize_int8, load_library,  # noqa: F401
                      mqa_decode, mqa_decode_noalloc, mqa_decode_append, mqa_decode_workspace_bytes, mqa_prefill_chunk,
                      mqa_status_string, default_softmax_scale, library_path,
                      decode_workspace, mqa_prefill_workspace_bytes, prefill_workspace,
                      PagedKV, kv_quantize_int8_paged, mqa_decode_paged, mqa_decode_append_paged,
                      mqa_decode_paged_workspace_bytes, mqa_prefill_chunk_paged, mqa_decode_q8,
                      mqa_decode_append_q8, mqa_decode_ragged, mqa_decode_append_ragged,
                      mqa_decode_ragged_workspace_bytes, ragged_workspace, PrefixCache, host_pool, kv_block_bytes,
                      mqa_kv_blocks_to_host, mqa_kv_blocks_to_device, mqa_set_deterministic)
