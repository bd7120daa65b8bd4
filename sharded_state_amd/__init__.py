"""sharded_state_amd -- the one-device data-parallel hot path of Fully Sharded
Data Parallel (ZeRO stage 3) on AMD Instinct MI355X (gfx950).

The pipeline of one FSDP unit per training step -- flatten + pad, emulated
reduce-scatter of N ranks' gradients, sharded AdamW on the fp32 master shard,
cast to the compute dtype, all-gather unshard, per-tensor views -- runs in the
hand-written HIP kernels of ``libfsdp_shard.so`` behind the C ABI declared in
``include/fsdp_shard.h``.  This package is its Python binding: argument
marshalling over ctypes, with PyTorch for device memory and streams.
"""
from ._native import AdamWHP, FsdpError, MAX_WORLD, OptimHP, lib  # noqa: F401
from .api import (  # noqa: F401
    dtype_code,
    fsdp_flatten_pad,
    fsdp_layout,
    fsdp_reduce_scatter_local,
    fsdp_sharded_adamw,
    fsdp_step_unit,
    fsdp_step_units,
    prepare_step_units,
    fsdp_unflatten_views,
    fsdp_unshard_gather,
    unit_gather_split,
    units_in_launch,
    view_table,
)
from .state import RankState  # noqa: F401
from .offload import (  # noqa: F401
    OffloadState,
    fsdp_host_adamw,
    fsdp_offload_step,
    fsdp_offload_step_units,
    fsdp_offload_step_units_noalloc,
    prepare_offload_step_units,
)
from .checkpoint import consolidate, load_shard, save_shard, shard_info, shard_path  # noqa: F401
from .config import UnitConfig, from_bf16_mixed_precision, from_fairseq  # noqa: F401

__all__ = [
    "AdamWHP", "OptimHP", "FsdpError", "MAX_WORLD", "lib", "dtype_code", "fsdp_layout", "fsdp_flatten_pad",
    "fsdp_reduce_scatter_local", "fsdp_sharded_adamw", "fsdp_step_unit", "fsdp_step_units", "prepare_step_units", "fsdp_unshard_gather",
    "fsdp_unflatten_views", "view_table", "RankState", "save_shard", "load_shard", "shard_info",
    "shard_path", "consolidate", "fsdp_host_adamw", "fsdp_offload_step", "fsdp_offload_step_units",
    "fsdp_offload_step_units_noalloc", "prepare_offload_step_units", "OffloadState", "unit_gather_split", "units_in_launch",
    "UnitConfig", "from_fairseq", "from_bf16_mixed_precision",
]
