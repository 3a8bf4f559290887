"""ZeRO-3 / FSDP shard step for AMD MI355X (gfx950).

One data-parallel rank's shard step, with D ranks simulated in one GPU's
memory: pack a unit into D shards, reduce-scatter arithmetic, fused
mixed-precision AdamW on the shard, and the all-gather's local rebuild.
The work runs in the HIP kernels of libzs.so; this package is its binding.
"""
from ._binding import (  # noqa: F401
    AdamWHP, LIB_PATH, ZS_BF16, ZS_EALIAS, ZS_EHIP, ZS_EINVAL, ZS_EUNSUPPORTED, ZS_F32,
    ZS_MAX_D, ZS_OK, ZsError, load, raw_adamw_step, zs_abi_version, zs_adamw_step,
    zs_adamw_step_ex, zs_reduce_shard_ex,
    zs_gather_unit, zs_last_error, zs_pack_flat, zs_reduce_shard, zs_step_pipelined,
    zs_unit_layout, zs_reshard, zs_shard_save, zs_shard_info_read, zs_shard_load,
    zs_shard_load_resharded, ZS_EIO, zs_adamw_step_host, zs_offload_step, zs_stream_ceiling,
    zs_hbm_probe, ZS_PROBE_READ, ZS_PROBE_WRITE, ZS_PROBE_COPY, ZS_PROBE_TRIAD, PackTable,
    zs_step_pipelined_static, ZS_W_STREAM, ZS_W_KEEP, zs_adamw_step_timed,
    zs_stream_ceiling_timed,
)

__all__ = [
    "zs_unit_layout", "zs_pack_flat", "zs_reduce_shard", "zs_adamw_step",
    "zs_reduce_shard_ex", "zs_adamw_step_ex", "zs_adamw_step_timed", "zs_reshard",
    "zs_shard_save", "zs_shard_info_read", "zs_shard_load", "zs_shard_load_resharded", "zs_adamw_step_host",
    "zs_offload_step", "zs_stream_ceiling", "zs_stream_ceiling_timed", "zs_hbm_probe",
    "ZS_PROBE_READ", "ZS_PROBE_WRITE", "ZS_PROBE_COPY", "ZS_PROBE_TRIAD",
    "zs_gather_unit", "zs_step_pipelined", "zs_last_error", "zs_abi_version", "AdamWHP", "ZsError",
    "ZS_BF16", "ZS_F32", "ZS_MAX_D", "load", "PackTable", "zs_step_pipelined_static",
]
