"""One unit's step configuration from the flags the pages give.

Two sources fix what a unit step computes besides its hyper-parameters:

* fairseq's FSDP flags and the ``fsdp_config`` they become ("fairseq 中的
  Fully Sharded Data Parallel (FSDP) 实战指南", "参数定义与底层实现" and
  "限制与兼容性说明"): reshard after forward is the negation of
  --no-reshard-after-forward; mixed precision is --fp16 without
  --memory-efficient-fp16; the compute dtype is fp16 with --fp16, else fp32;
  --fp32-reduce-scatter reduces in fp32 (default off); --cpu-offload needs
  --ddp-backend=fully_sharded and --fp16; the optimizer must be pointwise;
  BMUF is refused; FSDP relies on flattening.
* bf16 mixed precision ("FSDP (Fully Sharded Data Parallel)", "Mixed Precision
  and FSDP"): bf16 parameters for the forward with an fp32 master and fp32
  optimizer state, or pure bf16 without the master; resharding after the
  forward makes two all-gathers per step ("The Per-Layer Communication").

``UnitConfig`` holds the result: world, rank, gradient / state / compute dtypes,
fp32 reduce-scatter, gathers per step, CPU offload and the optimizer.  Host
logic only; ``step`` checks a unit table against the configuration and then
issues ``fsdp_step_units``.
"""
from dataclasses import dataclass

import torch

from . import _native as N
from .api import fsdp_step_units

# the pages' pointwise optimizers (compatible) and their examples of others (not)
POINTWISE = ("adam", "adamw", "adadelta", "adamax", "sgd")
NOT_POINTWISE = ("adagrad", "adafactor", "lamb")
_DTYPES = (torch.float32, torch.float16, torch.bfloat16)


@dataclass(frozen=True)
class UnitConfig:
    """What one unit step computes, apart from its hyper-parameters.

    grad_dtype:    each rank's flat gradient buffer
    state_dtype:   master parameter shard and optimizer state (float32, or the
                   16-bit compute dtype when there is no fp32 master)
    compute_dtype: the compute copy that is gathered
    fp32_reduce_scatter: reduce the gradients in fp32
    reshard_after_forward: parameters are freed after the forward and gathered
                   again for the backward (two all-gathers per step)
    cpu_offload:   master and optimizer state live in host memory
    optimizer:     a pointwise optimizer by name
    """
    world: int
    rank: int
    grad_dtype: torch.dtype
    state_dtype: torch.dtype
    compute_dtype: torch.dtype
    fp32_reduce_scatter: bool = False
    reshard_after_forward: bool = True
    cpu_offload: bool = False
    optimizer: str = "adamw"

    def __post_init__(self):
        if not 1 <= self.world <= N.MAX_WORLD:
            raise ValueError("world = %d outside [1, %d]" % (self.world, N.MAX_WORLD))
        if not 0 <= self.rank < self.world:
            raise ValueError("rank = %d outside [0, %d)" % (self.rank, self.world))
        for name in ("grad_dtype", "state_dtype", "compute_dtype"):
            if getattr(self, name) not in _DTYPES:
                raise ValueError("%s must be float32, float16 or bfloat16" % name)
        if self.state_dtype != torch.float32 and self.state_dtype != self.compute_dtype:
            raise ValueError("16-bit state is the compute copy itself: state_dtype must equal compute_dtype")
        if self.cpu_offload and self.state_dtype != torch.float32:
            raise ValueError("CPU offload keeps an fp32 master and fp32 optimizer state in host memory")
        if self.optimizer not in POINTWISE:
            raise ValueError("optimizer %r is not pointwise; sharded state needs one of %s"
                             % (self.optimizer, ", ".join(POINTWISE)))

    @property
    def gathers(self) -> int:
        """All-gathers of the unit per step."""
        return 2 if self.reshard_after_forward else 1

    @property
    def reduce_dtype(self) -> torch.dtype:
        """Precision of the reduce-scatter and of the averaged gradient shard."""
        return torch.float32 if (self.fp32_reduce_scatter or self.grad_dtype == torch.float32) else self.grad_dtype

    @property
    def mixed_precision(self) -> bool:
        """An fp32 master with a 16-bit compute copy."""
        return self.state_dtype == torch.float32 and self.compute_dtype != torch.float32

    def check_units(self, units):
        """Raise ValueError unless every unit of an ``fsdp_step_units`` table
        matches this configuration: N gradient buffers of grad_dtype, master
        (and kept state) of state_dtype, a full buffer of compute_dtype and N
        shards; with two gathers per step and an fp32 master, a persistent
        compute shard for the second all-gather.  No device work."""
        if not units:
            raise ValueError("units is empty")
        for k, u in enumerate(units):
            grads = u["rank_grads"]
            if len(grads) != self.world:
                raise ValueError("units[%d] has %d ranks, the configuration %d" % (k, len(grads), self.world))
            for q, g in enumerate(grads):
                if g.dtype != self.grad_dtype:
                    raise ValueError("units[%d].rank_grads[%d] is %s, the configuration %s"
                                     % (k, q, g.dtype, self.grad_dtype))
            for name in ("master", "exp_avg", "exp_avg_sq"):
                t = u.get(name)
                if t is not None and t.dtype != self.state_dtype:
                    raise ValueError("units[%d].%s is %s, the configuration %s" % (k, name, t.dtype, self.state_dtype))
            full = u.get("full")
            if full is None:
                raise ValueError("units[%d] has no full buffer: the step all-gathers" % k)
            if full.dtype != self.compute_dtype:
                raise ValueError("units[%d].full is %s, the configuration %s" % (k, full.dtype, self.compute_dtype))
            if full.numel() != self.world * u["master"].numel():
                raise ValueError("units[%d].full must hold world x shard elements" % k)
            if self.gathers == 2 and self.state_dtype == torch.float32 and u.get("compute_shard") is None:
                raise ValueError("units[%d]: with reshard after forward the second all-gather reads a persistent "
                                 "compute shard (compute_shard)" % k)

    def step(self, units, hp, stream=None):
        """``fsdp_step_units`` on a table checked against this configuration
        (the first all-gather of the step; with two gathers per step the
        caller gathers again from the shards after the forward)."""
        if self.cpu_offload:
            raise ValueError("a CPU-offload configuration steps through OffloadState")
        self.check_units(units)
        return fsdp_step_units(units, self.rank, self.fp32_reduce_scatter, hp, stream)


def from_fairseq(world, rank, *, ddp_backend="fully_sharded", fp16=False, memory_efficient_fp16=False,
                 no_reshard_after_forward=False, fp32_reduce_scatter=False, cpu_offload=False,
                 not_fsdp_flatten_parameters=False, optimizer="adam", use_bmuf=False):
    """The configuration fairseq's flags give, with its checks.

    Gradients are kept in the compute dtype.  With --memory-efficient-fp16
    mixed precision is off: the pages do not fix the state layout then; the
    library's form without an fp32 master (fp16 parameter, m and v) is the one
    returned."""
    if ddp_backend != "fully_sharded":
        if cpu_offload:
            raise ValueError("--cpu-offload requires --ddp-backend=fully_sharded")
        raise ValueError("sharded state needs --ddp-backend=fully_sharded, got %r" % ddp_backend)
    if use_bmuf:
        raise ValueError("--ddp-backend=fully_sharded is not compatible with --use-bmuf")
    if memory_efficient_fp16 and not fp16:
        raise ValueError("--memory-efficient-fp16 requires --fp16")
    if cpu_offload and not fp16:
        raise ValueError("--cpu-offload requires --fp16 (mixed precision)")
    if not_fsdp_flatten_parameters:
        raise ValueError("FSDP steps flat units: --not-fsdp-flatten-parameters is not supported")
    if optimizer in NOT_POINTWISE or optimizer not in POINTWISE:
        raise ValueError("optimizer %r is not pointwise; FSDP supports %s" % (optimizer, ", ".join(POINTWISE)))
    compute = torch.float16 if fp16 else torch.float32
    mixed = fp16 and not memory_efficient_fp16
    state = torch.float32 if (mixed or not fp16) else torch.float16
    return UnitConfig(world=world, rank=rank, grad_dtype=compute, state_dtype=state, compute_dtype=compute,
                      fp32_reduce_scatter=bool(fp32_reduce_scatter),
                      reshard_after_forward=not no_reshard_after_forward, cpu_offload=bool(cpu_offload),
                      optimizer=optimizer)


def from_bf16_mixed_precision(world, rank, *, fp32_master=True, reshard_after_forward=True,
                              fp32_reduce_scatter=False, optimizer="adamw"):
    """bf16 parameters and gradients for the forward and backward, with an fp32
    master and fp32 optimizer state, or pure bf16 (parameter, m and v in bf16)
    without the master."""
    return UnitConfig(world=world, rank=rank, grad_dtype=torch.bfloat16,
                      state_dtype=torch.float32 if fp32_master else torch.bfloat16,
                      compute_dtype=torch.bfloat16, fp32_reduce_scatter=bool(fp32_reduce_scatter),
                      reshard_after_forward=bool(reshard_after_forward), optimizer=optimizer)
