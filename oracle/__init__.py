"""fp64 CPU oracle for the SnapStream hot path.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its binding.
"""
from .snapstream_oracle import (  # noqa: F401
    CacheState,
    Config,
    PrefillResult,
    attend,
    decode_step,
    decode_write,
    fixed_cache_layout,
    max_pool_clipped,
    obs_column_scores,
    prefill_compress_one,
    ring_slot,
    rope_inv_freq,
    rope_rotate,
    round_to_bf16,
    round_to_dtype,
    select_topk,
)
