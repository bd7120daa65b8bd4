"""GPU parity of the CPU-offload step (fsdp_offload_step): device
reduce-scatter, chunked copy of the gradient shard to pinned host memory,
AdamW on the host-resident fp32 master/m/v, copy of the compute shard back to
the device.  Every simulated rank is stepped; master, m, v, the compute shards
and the gathered full buffer must equal the oracle bit for bit, and equal the
device-resident path (fsdp_sharded_adamw) on the same inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import sharded_state_amd as ss
from parity import assert_bits_equal, oracle_rank_step_threaded, UnitRun, assert_bitexact, assert_rel, compare_compute, np_of
from workloads import CONFIGS, gpt_block, llama_block, rank_grad, scaled

pytestmark = pytest.mark.gpu


def _offload_all_ranks(run, chunk, threads, copy_stream=None):
    c, S = run.cfg, run.S
    flat = ss.fsdp_flatten_pad(run.params, c.world)
    full = torch.empty(c.world * S, dtype=run.cdt_torch, device="cuda")
    states = []
    for r in range(c.world):
        sl = slice(r * S, (r + 1) * S)
        st = ss.OffloadState(flat[sl], run.grads[0].dtype, c.fp32_reduce, run.cdt_torch, "cuda",
                             exp_avg=run.m0[sl], exp_avg_sq=run.v0[sl])
        st.step(run.grads, r, run.hp(), full[sl], chunk_numel=chunk, n_threads=threads, copy_stream=copy_stream)
        states.append(st)
    torch.cuda.synchronize()
    return states, full


@pytest.mark.parametrize("base,shape,chunk,threads,copy_stream", [
    ("gpt2-large-block", gpt_block(64), 10_000, 4, False),      # N = 2, fp16 grads, fp32 reduce
    ("gpt3-13b-block", gpt_block(80), 12_344, 16, True),        # N = 8, shard not 16-byte aligned
    ("llama70b-block", llama_block(64, 80, 224), 0, 3, True),   # bf16 grads and reduce, one chunk
    ("gpt2-xl-model", gpt_block(48), 4_104, 1, False),          # bf16, 1 % zeros, many chunks
    ("tiny", [("t", (1001,)), ("u", (7,))], 16, 2, True),       # fp32 grads, ragged chunks of 16
])
def test_offload_step_matches_oracle_and_device_path(base, shape, chunk, threads, copy_stream):
    print("case", base, chunk, threads, copy_stream, flush=True)
    cfg = scaled(CONFIGS[base], shape)
    run = UnitRun(cfg)
    run.run_gpu()
    run.run_oracle()
    run.compare()
    cs = torch.cuda.Stream() if copy_stream else None
    states, full = _offload_all_ranks(run, chunk, threads, cs)
    S = run.S
    for r, st in enumerate(states):
        sl = slice(r * S, (r + 1) * S)
        for name, got, ref, dev in (("master", st.master, run.o_master, run.master),
                                    ("exp_avg", st.exp_avg, run.o_m, run.m),
                                    ("exp_avg_sq", st.exp_avg_sq, run.o_v, run.v)):
            g = np_of(got)
            assert_rel(g, ref[sl], "offload %s rank %d" % (name, r))
            assert_bitexact(g, ref[sl], "offload %s rank %d (bit-exact)" % (name, r))
            assert_bitexact(g, np_of(dev[sl]), "offload vs device %s rank %d" % (name, r))
        assert_bitexact(np_of(st.grad_host), run.o_gshard[r], "gradient shard on the host, rank %d" % r)
    f = np_of(full)
    compare_compute(f, run.o_full, cfg.compute_dt, "offload compute shards")
    assert_bitexact(f, run.o_full, "offload compute shards (bit-exact)")
    assert_bitexact(f, np_of(run.full), "offload vs device compute shards")
    gathered = ss.fsdp_unshard_gather([full[r * S:(r + 1) * S].clone() for r in range(cfg.world)])
    torch.cuda.synchronize()
    assert_bitexact(np_of(gathered), run.o_full, "gather of offloaded compute shards")


@pytest.mark.parametrize("copy_stream", [False, True])
def test_offload_batch_of_units_matches_oracle(copy_stream):
    """Five distinct units of different sizes (one empty) stepped by one
    fsdp_offload_step_units call, small chunks so that chunks of several units
    are in flight at once; each unit against the oracle, and the compute shards
    read on the stream right after the call (the ordering the call promises)."""
    base = CONFIGS["gpt3-13b-block"]
    shapes = [gpt_block(40), gpt_block(24), [("x", (999, 37))], [("e", (0,))], llama_block(32, 48, 96)]
    runs, units, outs, copies = [], [], [], []
    cs = torch.cuda.Stream() if copy_stream else None
    for k, shape in enumerate(shapes):
        run = UnitRun(scaled(base, shape, world=4), block=k)
        S = run.S
        flat = ss.fsdp_flatten_pad(run.params, 4)
        st = ss.OffloadState(flat[2 * S:3 * S], run.grads[0].dtype, run.cfg.fp32_reduce, run.cdt_torch, "cuda",
                             exp_avg=run.m0[2 * S:3 * S], exp_avg_sq=run.v0[2 * S:3 * S])
        out = torch.full((S,), float("nan"), dtype=run.cdt_torch, device="cuda")
        runs.append(run)
        units.append((st, run.grads, out))
        outs.append(out)
    torch.cuda.synchronize()
    ss.fsdp_offload_step_units(units, 2, base.fp32_reduce, runs[0].hp(), chunk_numel=3000, n_threads=6,
                               copy_stream=cs)
    copies = [o.clone() for o in outs]              # on the current stream, no synchronization before
    torch.cuda.synchronize()
    for k, (run, (st, _, out)) in enumerate(zip(runs, units)):
        run.run_oracle()
        S = run.S
        sl = slice(2 * S, 3 * S)
        assert_bitexact(np_of(st.master), run.o_master[sl], "unit %d master" % k)
        assert_bitexact(np_of(st.exp_avg), run.o_m[sl], "unit %d exp_avg" % k)
        assert_bitexact(np_of(st.exp_avg_sq), run.o_v[sl], "unit %d exp_avg_sq" % k)
        assert_bitexact(np_of(copies[k]), run.o_compute[2], "unit %d compute shard" % k)


def test_offload_batch_rejects_a_unit_twice():
    run = UnitRun(scaled(CONFIGS["gpt2-large-block"], gpt_block(16)))
    S = run.S
    st = ss.OffloadState(ss.fsdp_flatten_pad(run.params, 2)[:S], run.grads[0].dtype, True, run.cdt_torch, "cuda")
    outs = [torch.empty(S, dtype=run.cdt_torch, device="cuda") for _ in range(2)]
    with pytest.raises(ss.FsdpError, match="overlap"):
        ss.fsdp_offload_step_units([(st, run.grads, outs[0]), (st, run.grads, outs[1])], 0, True, run.hp())


def test_offload_two_steps_then_device_step_agree():
    """Step 1 and 2 offloaded vs on the device: the host state after two steps
    equals the device state after two steps."""
    cfg = scaled(CONFIGS["gpt3-13b-block"], gpt_block(40), world=4)
    run = UnitRun(cfg)
    S, r = run.S, 1
    sl = slice(r * S, (r + 1) * S)
    flat = ss.fsdp_flatten_pad(run.params, cfg.world)
    st = ss.OffloadState(flat[sl], run.grads[0].dtype, cfg.fp32_reduce, run.cdt_torch, "cuda",
                         exp_avg=run.m0[sl], exp_avg_sq=run.v0[sl])
    dev = [flat[sl].clone(), run.m0[sl].clone(), run.v0[sl].clone()]
    cd = torch.empty(S, dtype=run.cdt_torch, device="cuda")
    co = torch.empty(S, dtype=run.cdt_torch, device="cuda")
    for t in (1, 2):
        grads = run.grads if t == 1 else [g.flip(0).contiguous() for g in run.grads]
        st.step(grads, r, run.hp(t), co, chunk_numel=5000, n_threads=4)
        ss.fsdp_sharded_adamw(*dev, grads, r, cfg.fp32_reduce, run.hp(t), compute_shard=cd)
    torch.cuda.synchronize()
    for a, b, what in ((st.master, dev[0], "master"), (st.exp_avg, dev[1], "m"), (st.exp_avg_sq, dev[2], "v")):
        assert_bitexact(np_of(a), np_of(b), what)
    assert_bitexact(np_of(co), np_of(cd), "compute")


def test_offload_full_size_70b_block_every_element():
    """The 70B-shaped block at full size, rank 0 and rank 7, offloaded with the
    default chunks and 16 threads: every element of the host master, m and v
    and of the device compute shard against the oracle (run over disjoint
    chunks on all host threads)."""
    cfg = CONFIGS["llama70b-block"]
    world = cfg.world
    P, Pp, S = ss.fsdp_layout(cfg.numels, world)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    grads = [rank_grad(cfg, 0, q, Pp, "cuda") for q in range(world)]
    h = oracle.hp()
    for r in (0, world - 1):
        print("rank", r, flush=True)
        master = (torch.randn(S, device="cuda", generator=g) * 0.02)
        st = ss.OffloadState(master, grads[0].dtype, cfg.fp32_reduce, torch.bfloat16, "cuda")
        p, m, v = np_of(st.master), np.zeros(S, np.float32), np.zeros(S, np.float32)
        gs = [np_of(x[r * S:(r + 1) * S]) for x in grads]
        out = torch.empty(S, dtype=torch.bfloat16, device="cuda")
        st.step(grads, r, ss.AdamWHP(), out)
        torch.cuda.synchronize()
        _, comp = oracle_rank_step_threaded(gs, p, m, v, h, "bf16", cfg.fp32_reduce, "bf16")
        assert_bits_equal(np_of(st.master), p, "master rank %d" % r)
        assert_bits_equal(np_of(st.exp_avg), m, "exp_avg rank %d" % r)
        assert_bits_equal(np_of(st.exp_avg_sq), v, "exp_avg_sq rank %d" % r)
        assert_bits_equal(np_of(out), comp, "compute shard rank %d" % r)
        del st


def test_offload_rejects_bad_arguments():
    cfg = scaled(CONFIGS["tiny"], [("t", (64,))])
    run = UnitRun(cfg)
    S = run.S
    flat = ss.fsdp_flatten_pad(run.params, cfg.world)
    st = ss.OffloadState(flat[:S], run.grads[0].dtype, cfg.fp32_reduce, run.cdt_torch, "cuda")
    with pytest.raises(ss.FsdpError):
        st.step(run.grads, 0, ss.AdamWHP(step=0), torch.empty(S, dtype=run.cdt_torch, device="cuda"))
    assert st.grad_dev.dtype == run.cdt_torch == torch.float32
    with pytest.raises(ss.FsdpError, match="overlap"):    # compute shard on top of the gradient shard
        st.step(run.grads, 0, ss.AdamWHP(), st.grad_dev)
    with pytest.raises(ValueError):
        st.step(run.grads, 0, ss.AdamWHP(), torch.empty(S + 1, dtype=run.cdt_torch, device="cuda"))
