"""One rank's persistent sharded state of an FSDP unit.

Per-worker memory is the point of full sharding: a rank keeps only its shard of
every persistent class -- fp32 master weights, AdamW's m and v, the compute
copy and the reduce-scattered gradient -- so each class takes 1/N of the
unsharded unit plus the tail padding ("FSDP (Fully Sharded Data Parallel)",
section "The Sharding Scheme"; "Data Parallelism", section "ZeRO Stages").
This class allocates those buffers (device memory through torch); the pipeline
itself runs in libfsdp_shard.so.
"""
import torch

from .api import fsdp_layout

_SIZE = {torch.float32: 4, torch.float16: 2, torch.bfloat16: 2}


class RankState:
    """Buffers of rank `rank` for a unit with tensor sizes `numels`.

    master, exp_avg, exp_avg_sq : fp32, S elements (S = padded numel / world)
    compute                     : compute dtype, S elements
    grad_shard                  : reduce-scatter output, S elements of
                                  grad_shard_dtype (None: not kept)
    """

    def __init__(self, numels, world, rank, compute_dtype, grad_shard_dtype=None, device="cuda"):
        if not 0 <= rank < world:
            raise ValueError("rank %d outside [0, %d)" % (rank, world))
        self.numel, self.padded_numel, self.shard_numel = fsdp_layout(numels, world)
        self.world, self.rank = world, rank
        S = self.shard_numel
        self.master = torch.zeros(S, dtype=torch.float32, device=device)
        self.exp_avg = torch.zeros(S, dtype=torch.float32, device=device)
        self.exp_avg_sq = torch.zeros(S, dtype=torch.float32, device=device)
        self.compute = torch.empty(S, dtype=compute_dtype, device=device)
        self.grad_shard = (torch.empty(S, dtype=grad_shard_dtype, device=device)
                           if grad_shard_dtype is not None else None)

    def nbytes(self):
        """Bytes per persistent class: {"optimizer", "compute", "grad"}."""
        S = self.shard_numel
        out = {"optimizer": 12 * S, "compute": _SIZE[self.compute.dtype] * S}
        out["grad"] = _SIZE[self.grad_shard.dtype] * S if self.grad_shard is not None else 0
        return out
