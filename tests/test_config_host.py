"""The unit configuration from the pages' flags (host only, no GPU).

fairseq: "fairseq 中的 Fully Sharded Data Parallel (FSDP) 实战指南", sections
"参数定义与底层实现" (flag defaults and the fsdp_config mapping) and
"限制与兼容性说明" (pointwise optimizers only, no BMUF, flattening required,
--cpu-offload needs --ddp-backend=fully_sharded), and its single-GPU example
(--cpu-offload needs --fp16).  bf16: "FSDP (Fully Sharded Data Parallel)",
"Mixed Precision and FSDP" and "The Per-Layer Communication".
"""
import pytest
import torch

import sharded_state_amd as ss
import workloads

F32, F16, BF16 = torch.float32, torch.float16, torch.bfloat16


def test_fairseq_defaults():
    """Every flag at its default: fp32 compute, no fp32 reduce-scatter, reshard
    after forward (two all-gathers per step), no offload."""
    c = ss.from_fairseq(8, 3)
    assert (c.world, c.rank) == (8, 3)
    assert (c.grad_dtype, c.state_dtype, c.compute_dtype) == (F32, F32, F32)
    assert c.fp32_reduce_scatter is False and c.reshard_after_forward is True and c.gathers == 2
    assert c.cpu_offload is False and c.mixed_precision is False and c.reduce_dtype == F32


def test_fairseq_fp16_is_mixed_precision():
    """compute_dtype = fp16 with --fp16; mixed_precision = fp16 and not
    memory_efficient_fp16: an fp32 master under an fp16 compute copy."""
    c = ss.from_fairseq(2, 0, fp16=True)
    assert (c.grad_dtype, c.state_dtype, c.compute_dtype) == (F16, F32, F16)
    assert c.mixed_precision and c.reduce_dtype == F16
    assert ss.from_fairseq(2, 0, fp16=True, fp32_reduce_scatter=True).reduce_dtype == F32


def test_fairseq_no_reshard_after_forward_negates():
    assert ss.from_fairseq(2, 0).reshard_after_forward is True
    c = ss.from_fairseq(2, 0, no_reshard_after_forward=True)
    assert c.reshard_after_forward is False and c.gathers == 1


def test_fairseq_memory_efficient_fp16():
    """It requires --fp16 and turns mixed precision off (no fp32 master)."""
    with pytest.raises(ValueError, match="requires --fp16"):
        ss.from_fairseq(2, 0, memory_efficient_fp16=True)
    c = ss.from_fairseq(2, 0, fp16=True, memory_efficient_fp16=True)
    assert c.mixed_precision is False and (c.state_dtype, c.compute_dtype) == (F16, F16)


def test_fairseq_cpu_offload_checks():
    with pytest.raises(ValueError, match="--cpu-offload requires --ddp-backend=fully_sharded"):
        ss.from_fairseq(1, 0, ddp_backend="pytorch_ddp", fp16=True, cpu_offload=True)
    with pytest.raises(ValueError, match="requires --fp16"):
        ss.from_fairseq(1, 0, cpu_offload=True)
    c = ss.from_fairseq(1, 0, fp16=True, cpu_offload=True)
    assert c.cpu_offload and c.state_dtype == F32
    with pytest.raises(ValueError, match="OffloadState"):
        c.step([], ss.AdamWHP())


@pytest.mark.parametrize("name", ["adam", "adamw", "adadelta", "adamax", "sgd"])
def test_fairseq_pointwise_optimizers_accepted(name):
    assert ss.from_fairseq(2, 0, optimizer=name).optimizer == name


@pytest.mark.parametrize("name", ["adagrad", "adafactor", "lamb"])
def test_fairseq_non_pointwise_optimizers_refused(name):
    with pytest.raises(ValueError, match="not pointwise"):
        ss.from_fairseq(2, 0, optimizer=name)


def test_fairseq_refuses_bmuf_other_backends_and_unflattened_units():
    with pytest.raises(ValueError, match="bmuf"):
        ss.from_fairseq(2, 0, use_bmuf=True)
    with pytest.raises(ValueError, match="fully_sharded"):
        ss.from_fairseq(2, 0, ddp_backend="c10d")
    with pytest.raises(ValueError, match="flat"):
        ss.from_fairseq(2, 0, not_fsdp_flatten_parameters=True)


def test_bf16_mixed_precision_and_pure_bf16():
    c = ss.from_bf16_mixed_precision(8, 7)
    assert (c.grad_dtype, c.state_dtype, c.compute_dtype) == (BF16, F32, BF16) and c.mixed_precision
    assert c.gathers == 2
    p = ss.from_bf16_mixed_precision(8, 7, fp32_master=False, reshard_after_forward=False)
    assert (p.state_dtype, p.compute_dtype) == (BF16, BF16) and not p.mixed_precision and p.gathers == 1


def test_unit_config_rejects_inconsistent_settings():
    with pytest.raises(ValueError, match="rank"):
        ss.UnitConfig(world=2, rank=2, grad_dtype=F16, state_dtype=F32, compute_dtype=F16)
    with pytest.raises(ValueError, match="world"):
        ss.UnitConfig(world=129, rank=0, grad_dtype=F16, state_dtype=F32, compute_dtype=F16)
    with pytest.raises(ValueError, match="state_dtype must equal compute_dtype"):
        ss.UnitConfig(world=2, rank=0, grad_dtype=F16, state_dtype=BF16, compute_dtype=F16)
    with pytest.raises(ValueError, match="fp32 master"):
        ss.UnitConfig(world=2, rank=0, grad_dtype=BF16, state_dtype=BF16, compute_dtype=BF16, cpu_offload=True)
    with pytest.raises(ValueError, match="float32, float16 or bfloat16"):
        ss.UnitConfig(world=2, rank=0, grad_dtype=torch.float64, state_dtype=F32, compute_dtype=F16)


@pytest.mark.parametrize("name,make", [
    ("tiny", lambda w: ss.from_fairseq(w, 0, fp32_reduce_scatter=True, no_reshard_after_forward=True)),
    ("gpt2-large-block", lambda w: ss.from_fairseq(w, 0, fp16=True, fp32_reduce_scatter=True,
                                                    no_reshard_after_forward=True)),
    ("gpt2-xl-model", lambda w: ss.from_bf16_mixed_precision(w, 0, reshard_after_forward=False)),
    ("gpt3-13b-block", lambda w: ss.from_fairseq(w, 0, fp16=True, fp32_reduce_scatter=True)),
    ("llama70b-block", lambda w: ss.from_bf16_mixed_precision(w, 0, reshard_after_forward=False)),
])
def test_benchmark_workloads_are_these_flags(name, make):
    """Each benchmark workload is what its flags give: the same gradient,
    reduce and compute dtypes and all-gathers per step."""
    cfg = workloads.CONFIGS[name]
    c = make(cfg.world)
    assert c.grad_dtype == workloads.TORCH_DTYPE[cfg.grad_dt]
    assert c.compute_dtype == workloads.TORCH_DTYPE[cfg.compute_dt]
    assert c.reduce_dtype == (F32 if cfg.fp32_reduce else workloads.TORCH_DTYPE[cfg.grad_dt])
    assert c.gathers == cfg.gathers
    assert c.state_dtype == F32


def _unit(world, S, gdt, sdt, cdt, persistent):
    u = dict(master=torch.empty(S, dtype=sdt), exp_avg=torch.empty(S, dtype=sdt), exp_avg_sq=torch.empty(S, dtype=sdt),
             rank_grads=[torch.empty(world * S, dtype=gdt) for _ in range(world)],
             peer_shards=[torch.empty(S, dtype=cdt) for _ in range(world)], full=torch.empty(world * S, dtype=cdt))
    if persistent:
        u["compute_shard"] = torch.empty(S, dtype=cdt)
    return u


def test_check_units_against_the_configuration():
    """Host-side check of a unit table (CPU tensors: nothing reaches the device)."""
    c = ss.from_fairseq(2, 0, fp16=True, fp32_reduce_scatter=True)          # two gathers: persistent copy
    c.check_units([_unit(2, 64, F16, F32, F16, True)])
    with pytest.raises(ValueError, match="persistent"):
        c.check_units([_unit(2, 64, F16, F32, F16, False)])
    with pytest.raises(ValueError, match="rank_grads"):
        c.check_units([_unit(2, 64, BF16, F32, F16, True)])
    with pytest.raises(ValueError, match="master"):
        c.check_units([_unit(2, 64, F16, BF16, F16, True)])
    with pytest.raises(ValueError, match="full"):
        c.check_units([_unit(2, 64, F16, F32, BF16, True)])
    with pytest.raises(ValueError, match="ranks"):
        c.check_units([_unit(4, 64, F16, F32, F16, True)])
    one = ss.from_fairseq(2, 0, fp16=True, no_reshard_after_forward=True)
    one.check_units([_unit(2, 64, F16, F32, F16, False)])
