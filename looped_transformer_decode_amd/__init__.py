"""Looped Latent Attention decode hot path for AMD MI355X (gfx950).

The work runs in liblla.so (C ABI: include/lla.h); this package holds the
HIP sources (csrc/), the in-tree build, and a thin ctypes binding whose
functions carry the C entry points' names."""
from .lla import (LLA_2D, LLA_DT_BF16, LLA_DT_F32, LLA_PER_HEAD, EXPORTS, KvCache,
                  KvCacheDesc, LatentStore, LlaError, StoreDesc, kv_workspace, lib,
                  lla_kv_append, lla_kv_cache_bytes, lla_kv_cache_check, lla_kv_decode_attn,
                  lla_kv_decode_auto_splits, lla_kv_decode_workspace_bytes,
                  lla_kv_fill_from_store, lla_kv_rope_table_bytes, lla_kv_rope_table_fill,
                  lla2d_decode_attn, lla2d_encode_append,
                  lla_compression_ratio, lla_decode_attn, lla_decode_attn_inflight,
                  lla_decode_attn_noalloc, NOALLOC_SCRATCH_BYTES,
                  lla_decode_auto_splits, lla_decode_inflight_workspace_bytes, lla_decode_path,
                  lla_decode_workspace_bytes, lla_encode_append, lla_rope_table_bytes,
                  lla_rope_table_fill, lla_store_bytes, lla_store_check, lla_store_offset,
                  lla_svd_init, lla_svd_init_workspace_bytes, rope_table, status_string,
                  workspace)
