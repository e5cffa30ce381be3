"""MI355X-native attention-guided KV eviction and in-place paged compaction.

The compute lives in libkvs.so (HIP kernels for gfx950 behind the C ABI in
include/kvs.h); this package is its ctypes binding plus a round driver.
"""
from ._lib import (  # noqa: F401
    EXPORTS, KvsError, ObserverSet, PagedCache, SeqBatch, kvs_budget_ratchet, kvs_compact,
    kvs_lrfu_decay, kvs_lrfu_select, kvs_lrfu_update, kvs_pair_capacity, kvs_plan, kvs_plan_compact, kvs_score,
    kvs_score_workspace_size, kvs_select, kvs_version, lib, kvs_token_confidence,
    kvs_token_confidence_workspace_size, kvs_confidence_trend, KVS_DTYPE_F32, KVS_DTYPE_BF16,
    DecodeQueries, kvs_decode_workspace_size, kvs_decode_attention, StepSet, kvs_step_select_workspace_size,
    kvs_step_select, CacheShape, kvs_beacon_kmeans, kvs_beacon_seed, kvs_eviction_round,
    kvs_token_confidence_static, kvs_lrfu_select_compact,
)
from .round import RoundBuffers, eviction_round  # noqa: F401
