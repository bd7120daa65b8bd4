"""GPU parity: the HIP path through the C ABI against the oracle, element by
element, on seeded inputs with the dtypes and distributions of each workload,
at sizes the oracle finishes in seconds that still span many workgroups and a
ragged last tile; plus padding, unaligned and degenerate cases.
"""
import numpy as np
import pytest
import torch

import oracle
import sharded_state_amd as ss
from parity import (UnitRun, assert_bitexact, assert_rel, assert_ulp16, compare_compute, np_of)
from workloads import CONFIGS, gpt2_model, gpt_block, llama_block, scaled

pytestmark = pytest.mark.gpu


def _cases():
    C = CONFIGS
    return {
        "tiny": C["tiny"],                                                  # full size
        "gpt2-large-d96": scaled(C["gpt2-large-block"], gpt_block(96)),
        "gpt2-xl-d64": scaled(C["gpt2-xl-model"], gpt2_model(64, 2, 1000, 64)),
        "gpt3-13b-d128": scaled(C["gpt3-13b-block"], gpt_block(128)),
        "gpt3-13b-d80-unaligned": scaled(C["gpt3-13b-block"], gpt_block(80)),
        "llama70b-d64": scaled(C["llama70b-block"], llama_block(64, 80, 224)),
    }


CASES = _cases()


@pytest.mark.parametrize("name", list(CASES))
def test_unit_matches_oracle(name):
    print("case", name, flush=True)
    run = UnitRun(CASES[name])
    run.run_gpu()
    run.run_oracle()
    run.compare()


@pytest.mark.parametrize("name", list(CASES))
def test_step_unit_matches_oracle(name):
    """The one-launch unit step (fused reduce-scatter + AdamW + cast + gather)
    gives the oracle's results for every rank, and the same bytes as the
    two-call pipeline."""
    print("case", name, flush=True)
    run = UnitRun(CASES[name])
    run.run_gpu()
    run.run_oracle()
    run.compare()
    run.run_gpu_step_unit(persistent=name.startswith("gpt3"))
    run.compare_step_unit()


@pytest.mark.parametrize("P,world", [(1, 8), (7, 2), (9, 8), (9, 3), (1_000_001, 2),
                                     (1_000_001, 3), (1_000_001, 7), (4099, 1), (12345, 16)])
@pytest.mark.parametrize("base", ["gpt2-large-block", "llama70b-block"])
def test_padding_and_odd_world_sizes(P, world, base):
    print("case", base, P, world, flush=True)
    split = [P // 3, P - P // 3 - P // 5, P // 5]
    tensors = [("t%d" % i, (n,)) for i, n in enumerate(split) if n > 0]
    cfg = scaled(CONFIGS[base], tensors, world=world)
    run = UnitRun(cfg)
    run.run_gpu()
    run.run_oracle()
    run.compare()
    run.run_gpu_step_unit(persistent=True)
    run.compare_step_unit()
    pad = run.Pp - run.P
    assert not np.any(np_of(run.master)[run.P:].view(np.uint32))
    assert pad == oracle.padded_numel(P, world) - P


@pytest.mark.parametrize("S", [8, 504, 512, 520, 1024, 1032, 2552, 6664])
@pytest.mark.parametrize("base,world", [("gpt2-large-block", 2), ("llama70b-block", 8)])
def test_shards_around_whole_groups(S, base, world):
    """The unit kernel takes whole groups of 512 elements on the vector path and
    the rest (up to 519 elements) one element per lane: shards just under, at
    and just over multiples of 512 give the oracle's results."""
    print("case", base, S, world, flush=True)
    P = S * world
    tensors = [("t0", (P // 2,)), ("t1", (P - P // 2,))]
    cfg = scaled(CONFIGS[base], tensors, world=world)
    run = UnitRun(cfg)
    assert run.S == S
    run.run_gpu()
    run.run_oracle()
    run.compare()
    run.run_gpu_step_unit(persistent=True)
    run.compare_step_unit()


@pytest.mark.parametrize("step", [1, 10, 1000])
def test_later_steps(step):
    run = UnitRun(scaled(CONFIGS["gpt2-xl-model"], gpt_block(64)))
    run.run_gpu(step)
    run.run_oracle(step)
    run.compare()


def test_unaligned_buffers_take_the_scalar_path():
    """Views offset by one element defeat 16-byte alignment; results are the same."""
    g = torch.Generator().manual_seed(5)
    S, world = 5003, 2
    grads = [(torch.randn(world * S + 1, generator=g) * 1e-4).half().cuda() for _ in range(world)]
    gv = [x[1:] for x in grads]
    master = (torch.randn(S + 1, generator=g) * 0.02).cuda()
    m = torch.zeros(S + 1, device="cuda")
    v = torch.zeros(S + 1, device="cuda")
    out = torch.empty(S + 1, dtype=torch.float16, device="cuda")
    hp = ss.AdamWHP()
    p0 = np_of(master[1:])
    ss.fsdp_sharded_adamw(master[1:], m[1:], v[1:], gv, 1, True, hp, compute_shard=out[1:])
    torch.cuda.synchronize()
    gn = [np_of(x) for x in gv]
    p, mm, vv = p0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
    _, c = oracle.rank_step(gn, 1, p, mm, vv, oracle.hp(), "f16", True, "f16")
    assert_bitexact(np_of(master[1:]), p, "master")
    assert_bitexact(np_of(out[1:]), c, "compute")
    rs = ss.fsdp_reduce_scatter_local(gv, 1, False, out=torch.empty(S + 1, dtype=torch.float16,
                                                                    device="cuda")[1:], shard_numel=S)
    assert_bitexact(np_of(rs), oracle.reduce_scatter(gn, 1, "f16", False), "rs 16-bit")


@pytest.mark.parametrize("grad_dt,fp32_reduce", [("f16", True), ("f16", False), ("bf16", True), ("bf16", False)])
def test_reduce_scatter_of_rows_at_an_odd_stride(grad_dt, fp32_reduce):
    """Three ranks' gradients as the rows of one buffer whose row length, 3 S,
    is an odd number of 16-bit elements: rows 1 and 2 start 14 and 12 bytes past
    a 16-byte boundary, so every rank's reads take the per-element path for
    every row but the first; each rank's shard equals the oracle's, in fp32 and
    in 16-bit mode."""
    world, S = 3, 3 * 4096 + 517
    tdt = torch.float16 if grad_dt == "f16" else torch.bfloat16
    g = torch.Generator().manual_seed(17)
    rows = (torch.randn(world, world * S, generator=g) * 1e-3).to(tdt).cuda()
    assert (rows[1].data_ptr() - rows.data_ptr()) % 16 == 14 and (rows[2].data_ptr() - rows.data_ptr()) % 16 == 12
    grads = list(rows.unbind(0))
    host = [np_of(x) for x in grads]
    for rank in range(world):
        out = ss.fsdp_reduce_scatter_local(grads, rank, fp32_reduce)
        torch.cuda.synchronize()
        assert_bitexact(np_of(out), oracle.reduce_scatter(host, rank, grad_dt, fp32_reduce), "rank %d" % rank)


def test_unflatten_and_flatten_with_odd_offsets():
    """The tiny unit's last tensor is one element at an offset that is not a
    multiple of 4 elements; 16-bit tensors of odd sizes break 16-byte alignment."""
    g = torch.Generator().manual_seed(1)
    sizes = [1, 999, 3, 4097, 7, 1, 65536 + 5]
    for dt in (torch.float32, torch.bfloat16):
        ts = [(torch.randn(n, generator=g)).to(dt).cuda() for n in sizes]
        flat = ss.fsdp_flatten_pad(ts, 8)
        ref = oracle.flatten_pad([np_of(t) for t in ts], 8, "f32" if dt == torch.float32 else "bf16")
        torch.cuda.synchronize()
        assert_bitexact(np_of(flat), ref, "flatten")
        back = ss.fsdp_unflatten_views(flat, [(n,) for n in sizes], materialize=True)
        for a, b in zip(back, ts):
            assert torch.equal(a.view(torch.int16) if dt != torch.float32 else a.view(torch.int32),
                               b.view(torch.int16) if dt != torch.float32 else b.view(torch.int32))


def test_nan_and_inf_gradients_propagate_like_the_oracle():
    cfg = scaled(CONFIGS["gpt2-large-block"], gpt_block(32))
    run = UnitRun(cfg)
    for q, pos, val in ((0, 3, float("nan")), (1, 100, float("inf")), (0, 101, float("-inf")),
                        (1, 5000, 65504.0), (0, 5000, 65504.0)):
        run.grads[q][pos] = val
    run.run_gpu()
    run.run_oracle()
    run.compare()
    assert np.isnan(np_of(run.master)[3]) and np.isnan(np_of(run.master)[100])


def test_empty_shard_is_a_no_op():
    z = torch.empty(0, device="cuda")
    ss.fsdp_sharded_adamw(z, z.clone(), z.clone(), [torch.empty(0, dtype=torch.bfloat16, device="cuda")],
                          0, False, ss.AdamWHP())
    torch.cuda.synchronize()


def test_device_memory_exhaustion_raises_in_python_before_any_launch():
    """With torch's allocator capped below a rank's state, RankState raises
    torch.cuda.OutOfMemoryError in the Python layer (nothing is launched), and
    the library works as before once the cap is lifted."""
    print("case allocator cap", flush=True)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    total = torch.cuda.get_device_properties(0).total_memory
    torch.cuda.set_per_process_memory_fraction((1 << 30) / total)      # about 1 GiB
    try:
        with pytest.raises(torch.cuda.OutOfMemoryError):
            ss.RankState([1 << 30], 1, 0, torch.bfloat16)              # 4 GiB of fp32 master alone
    finally:
        torch.cuda.set_per_process_memory_fraction(1.0)
        torch.cuda.empty_cache()
    grads = [torch.randn(2 * 4099, device="cuda").half() for _ in range(2)]
    out = ss.fsdp_reduce_scatter_local(grads, 1, True)
    torch.cuda.synchronize()
    ref = oracle.reduce_scatter([np_of(g) for g in grads], 1, "f16", True)
    assert_bitexact(np_of(out), ref, "reduce-scatter after the cap")


def test_run_twice_is_bitwise_deterministic():
    cfg = scaled(CONFIGS["llama70b-block"], llama_block(64, 80, 224))
    a, b = UnitRun(cfg), UnitRun(cfg)
    a.run_gpu()
    b.run_gpu()
    for x, y in ((a.master, b.master), (a.m, b.m), (a.v, b.v), (a.full, b.full)):
        assert torch.equal(x.view(torch.int16) if x.dtype != torch.float32 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype != torch.float32 else y.view(torch.int32))


def test_fp16_16bit_reduce_and_fp32_compute_combinations():
    """Dtype combinations beyond the five workloads: fp16 grads reduced in 16
    bits, bf16 grads reduced in fp32, fp32 and bf16 compute copies."""
    for gd, fp32r, cd in (("f16", False, "f32"), ("bf16", True, "f16"), ("f32", True, "bf16")):
        cfg = scaled(CONFIGS["gpt2-large-block"], gpt_block(48), grad_dt=gd, fp32_reduce=fp32r,
                     compute_dt=cd, world=4)
        run = UnitRun(cfg)
        run.run_gpu()
        run.run_oracle()
        run.compare()


def _batch_units(runs, rank, gather=True):
    units = []
    for r in runs:
        world, S = r.cfg.world, r.S
        sl = slice(rank * S, (rank + 1) * S)
        u = dict(master=r.flat0[sl].clone(), exp_avg=r.m0[sl].clone(), exp_avg_sq=r.v0[sl].clone(),
                 rank_grads=r.grads)
        if gather:
            u["peer_shards"] = [None if q == rank else r.compute[q] for q in range(world)]
            u["full"] = torch.empty(world * S, dtype=r.cdt_torch, device="cuda")
        else:
            u["compute_shard"] = torch.empty(S, dtype=r.cdt_torch, device="cuda")
        units.append(u)
    return units


@pytest.mark.parametrize("base", ["tiny", "gpt2-large-block", "gpt2-xl-model", "gpt3-13b-block",
                                  "llama70b-block"])
def test_step_units_batch_matches_oracle(base):
    """Units of different sizes -- whole vectors, ragged tails, a single element,
    blocks that are not 16-byte aligned -- stepped together in one call give the
    oracle's bytes for every unit."""
    print("case", base, flush=True)
    shapes = [gpt_block(24), gpt_block(40), [("t", (1,))], [("t", (7,))], [("t", (1001,))], gpt_block(64)]
    runs = [UnitRun(scaled(CONFIGS[base], t, name="b%d" % i), block=i) for i, t in enumerate(shapes)]
    for r in runs:
        r.run_gpu()
        r.run_oracle()
        r.compare()
    world = runs[0].cfg.world
    for gather in (True, False):
        for rank in sorted({0, world - 1}):
            units = _batch_units(runs, rank, gather)
            ss.fsdp_step_units(units, rank, runs[0].cfg.fp32_reduce, runs[0].hp())
            torch.cuda.synchronize()
            for r, u in zip(runs, units):
                sl = slice(rank * r.S, (rank + 1) * r.S)
                assert_bitexact(np_of(u["master"]), r.o_master[sl], "master %s rank %d" % (r.cfg.name, rank))
                assert_bitexact(np_of(u["exp_avg"]), r.o_m[sl], "exp_avg %s" % r.cfg.name)
                assert_bitexact(np_of(u["exp_avg_sq"]), r.o_v[sl], "exp_avg_sq %s" % r.cfg.name)
                if gather:
                    assert_bitexact(np_of(u["full"]), np_of(r.full), "full %s rank %d" % (r.cfg.name, rank))
                else:
                    assert_bitexact(np_of(u["compute_shard"]), np_of(r.compute[rank]), "compute %s" % r.cfg.name)


def test_step_units_more_units_than_one_launch_holds():
    """70 units at N = 2 take two launches (40 + 30) and still match."""
    runs = [UnitRun(scaled(CONFIGS["gpt2-large-block"], [("t", (97 + 13 * i,))], name="u%d" % i), block=i)
            for i in range(70)]
    for r in runs:
        r.run_gpu()
        r.run_oracle()
    units = _batch_units(runs, 1)
    ss.fsdp_step_units(units, 1, True, runs[0].hp())
    torch.cuda.synchronize()
    for r, u in zip(runs, units):
        sl = slice(r.S, 2 * r.S)
        assert_bitexact(np_of(u["master"]), r.o_master[sl], "master %s" % r.cfg.name)
        assert_bitexact(np_of(u["full"]), np_of(r.full), "full %s" % r.cfg.name)


def test_step_units_rejects_a_unit_twice():
    run = UnitRun(scaled(CONFIGS["gpt2-large-block"], gpt_block(16)))
    run.run_gpu()
    u = _batch_units([run], 0)[0]
    with pytest.raises(ss.FsdpError) as e:
        ss.fsdp_step_units([u, u], 0, True, run.hp())
    assert e.value.code == -4
