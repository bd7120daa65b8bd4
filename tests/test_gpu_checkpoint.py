"""Sharded-state checkpoints of device-resident state on the GPU.

* save / load round trip bit for bit, fp32 and bf16 state, buffers spanning
  several 32 MB staging chunks;
* consolidation of the N shard files (gather + per-tensor views) equals the
  oracle's unflatten of its gathered master, m and v;
* resume: step t, save, load into fresh buffers, step t+1 gives the same bytes
  as stepping twice without the checkpoint.
"""
import numpy as np
import pytest
import torch

import oracle
import sharded_state_amd as ss
from parity import UnitRun, assert_bitexact, np_of
from workloads import CONFIGS, gpt_block, scaled

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_device_round_trip_over_several_chunks(tmp_path, dtype):
    S = 20_000_003                       # fp32: 80 MB per buffer, 3 staging chunks each
    world = 4
    numels = [S * world - 5, 3]
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    state = [(torch.randn(S, device="cuda", generator=g) * s).to(dtype) for s in (0.02, 1e-3, 1e-6)]
    path = ss.shard_path(str(tmp_path / "big"), 2)
    ss.save_shard(path, numels, world, 2, *state, step=11, hp=ss.AdamWHP())
    p, m, v, info = ss.load_shard(path)
    torch.cuda.synchronize()
    assert info["shard_numel"] == S and info["state_dtype"] == dtype and info["step"] == 11
    for a, b in zip(state, (p, m, v)):
        view = torch.int32 if dtype == torch.float32 else torch.int16
        assert torch.equal(a.view(view), b.view(view))


@pytest.mark.parametrize("base", ["gpt2-large-block", "llama70b-block"])
def test_consolidation_equals_oracle_unflatten(tmp_path, base):
    cfg = scaled(CONFIGS[base], gpt_block(48), world=4 if base == "gpt2-large-block" else 8)
    run = UnitRun(cfg)
    run.run_gpu()
    run.run_oracle()
    run.compare()
    S, world = run.S, cfg.world
    prefix = str(tmp_path / base)
    for r in range(world):
        sl = slice(r * S, (r + 1) * S)
        ss.save_shard(ss.shard_path(prefix, r), cfg.numels, world, r, run.master[sl], run.m[sl], run.v[sl],
                      step=1, hp=run.hp(), compute_dtype=run.cdt_torch)
    full = ss.consolidate(prefix, cfg.shapes)
    torch.cuda.synchronize()
    for key, ref in (("param", run.o_master), ("exp_avg", run.o_m), ("exp_avg_sq", run.o_v)):
        want = oracle.unflatten(ref, cfg.shapes, "f32")
        for k, (a, b) in enumerate(zip(full[key], want)):
            assert tuple(a.shape) == tuple(b.shape)
            assert_bitexact(np_of(a).reshape(-1), b.reshape(-1), "%s tensor %d" % (key, k))


def test_resume_from_a_shard_file_is_bitwise_continuous(tmp_path):
    cfg = scaled(CONFIGS["gpt3-13b-block"], gpt_block(64))
    run = UnitRun(cfg)
    S, world, rank = run.S, cfg.world, 3
    sl = slice(rank * S, (rank + 1) * S)
    flat = ss.fsdp_flatten_pad(run.params, world)
    a = [flat[sl].clone(), run.m0[sl].clone(), run.v0[sl].clone()]
    b = [x.clone() for x in a]
    for t in (1, 2):                                     # continuous
        ss.fsdp_sharded_adamw(*a, run.grads, rank, cfg.fp32_reduce, run.hp(t))
    ss.fsdp_sharded_adamw(*b, run.grads, rank, cfg.fp32_reduce, run.hp(1))
    path = ss.shard_path(str(tmp_path / "resume"), rank)
    ss.save_shard(path, cfg.numels, world, rank, *b, step=1, hp=run.hp(1))
    c = list(ss.load_shard(path)[:3])
    info, _ = ss.shard_info(path)
    ss.fsdp_sharded_adamw(*c, run.grads, rank, cfg.fp32_reduce, run.hp(info["step"] + 1))
    torch.cuda.synchronize()
    for x, y in zip(a, c):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
