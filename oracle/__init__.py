"""CPU oracle of the ZeRO-3 shard step (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product path never does.
"""
from .zs_oracle import (  # noqa: F401
    AdamWHP, BF16, FP32, adamw_constants, adamw_step, bf16_round, bf16_widen,
    bucket_bytes, bytes_per_device, gather_unit, pack_flat, rank_step,
    rank_step_hybrid, reduce_shard, reduce_shard_hybrid, reshard, round_to_dtype,
    transient_block_bytes, unit_layout, unit_views,
    zero3_steady_bytes,
)
