"""GPU parity of the pure 16-bit state variant: no fp32 master, the parameter,
m and v kept in bf16 (or fp16); the parameter shard is the compute shard.

Every simulated rank steps its shard through fsdp_step_units without the
gather, the full buffer is gathered from the updated parameter shards, and
then every rank steps again from the same initial state with the fused gather.
The oracle runs the same steps; results must match bit for bit (the bar for
16-bit outputs is 1 ulp).
"""
import numpy as np
import pytest
import torch

import oracle
import sharded_state_amd as ss
from parity import assert_bits_equal, oracle_chunks, assert_bitexact, assert_ulp16, dt_name, np_of
from workloads import CONFIGS, TORCH_DTYPE, gpt_block, llama_block, moments, param_tensors, rank_grad, scaled

pytestmark = pytest.mark.gpu


def _run(cfg, state_dt, step=1, block=0):
    sd = TORCH_DTYPE[state_dt]
    world = cfg.world
    P, Pp, S = ss.fsdp_layout(cfg.numels, world)
    params = [t.to(sd).cuda() for t in param_tensors(cfg, block)]          # 16-bit parameters
    grads = [rank_grad(cfg, block, q, Pp).cuda() for q in range(world)]
    m0, v0 = (x.to(sd).cuda() for x in moments(cfg, block, 0, Pp, P))
    hp = ss.AdamWHP(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, step)
    flat0 = ss.fsdp_flatten_pad(params, world)

    # GPU, pass 1: every rank without the gather, then gather the parameter shards
    p1, m1, v1 = flat0.clone(), m0.clone(), v0.clone()
    for r in range(world):
        sl = slice(r * S, (r + 1) * S)
        ss.fsdp_step_units([dict(master=p1[sl], exp_avg=m1[sl], exp_avg_sq=v1[sl], rank_grads=grads)], r,
                           cfg.fp32_reduce, hp)
    full1 = ss.fsdp_unshard_gather([p1[r * S:(r + 1) * S] for r in range(world)])
    # GPU, pass 2: every rank from the initial state with the fused gather
    fulls, states = [], []
    for r in range(world):
        sl = slice(r * S, (r + 1) * S)
        u = dict(master=flat0[sl].clone(), exp_avg=m0[sl].clone(), exp_avg_sq=v0[sl].clone(), rank_grads=grads,
                 peer_shards=[None if q == r else p1[q * S:(q + 1) * S] for q in range(world)],
                 full=torch.empty(world * S, dtype=sd, device="cuda"))
        ss.fsdp_step_units([u], r, cfg.fp32_reduce, hp)
        fulls.append(u["full"])
        states.append(u)
    torch.cuda.synchronize()

    # oracle
    o_flat = oracle.flatten_pad([np_of(t).reshape(-1) for t in params], world, state_dt)
    assert_bitexact(np_of(flat0), o_flat, "flatten (16-bit)")
    gs = [np_of(g) for g in grads]
    op, om, ov = o_flat.copy(), np_of(m0), np_of(v0)
    h = oracle.hp(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, step)
    for r in range(world):
        sl = slice(r * S, (r + 1) * S)
        p, m, v = op[sl].copy(), om[sl].copy(), ov[sl].copy()
        oracle.rank_step16(gs, r, p, m, v, h, dt_name(grads[0].dtype), cfg.fp32_reduce, state_dt)
        op[sl], om[sl], ov[sl] = p, m, v
    for name, got, ref in (("param", p1, op), ("exp_avg", m1, om), ("exp_avg_sq", v1, ov)):
        g = np_of(got)
        assert_ulp16(g, ref, state_dt, name)
        assert_bitexact(g, ref, name + " (bit-exact)")
    assert_bitexact(np_of(full1), op, "gathered parameters")
    for r in range(world):
        sl = slice(r * S, (r + 1) * S)
        assert_bitexact(np_of(fulls[r]), op, "fused gather, rank %d" % r)
        assert_bitexact(np_of(states[r]["master"]), op[sl], "fused param, rank %d" % r)
        assert_bitexact(np_of(states[r]["exp_avg_sq"]), ov[sl], "fused v, rank %d" % r)


@pytest.mark.parametrize("state_dt", ["bf16", "f16"])
@pytest.mark.parametrize("base,shape", [
    ("llama70b-block", llama_block(64, 80, 224)),
    ("gpt2-xl-model", gpt_block(48)),
    ("gpt3-13b-block", gpt_block(80)),            # N = 8 with a shard that is not 16-byte aligned
    ("gpt2-large-block", [("t", (1001,)), ("u", (7,))]),
])
def test_state16_matches_oracle(state_dt, base, shape):
    print("case", base, state_dt, flush=True)
    _run(scaled(CONFIGS[base], shape), state_dt)


def test_state16_later_step_and_odd_world():
    _run(scaled(CONFIGS["llama70b-block"], gpt_block(40), world=3), "bf16", step=100, block=3)


def test_state16_full_size_70b_block_every_element():
    """The 70B-shaped block at full size with bf16 state, rank 0 and rank 7,
    through the batched unit step with the fused gather: every element of the
    parameter, m and v shards and of the full buffer against the oracle (run
    over disjoint chunks on all host threads)."""
    cfg = CONFIGS["llama70b-block"]
    world = cfg.world
    P, Pp, S = ss.fsdp_layout(cfg.numels, world)
    sd = torch.bfloat16
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    flat = (torch.randn(Pp, device="cuda", generator=g) * 0.02).to(sd)
    flat[P:] = 0
    grads = [rank_grad(cfg, 0, q, Pp, "cuda") for q in range(world)]
    m = torch.zeros(Pp, dtype=sd, device="cuda")
    v = torch.zeros(Pp, dtype=sd, device="cuda")
    hp = ss.AdamWHP()
    peers = [(torch.randn(S, device="cuda", generator=g) * 0.02).to(sd) for _ in range(world)]
    h = oracle.hp()
    for r in (0, world - 1):
        print("rank", r, flush=True)
        sl = slice(r * S, (r + 1) * S)
        gs = [np_of(x[sl]) for x in grads]
        p0, m0, v0 = np_of(flat[sl]), np_of(m[sl]), np_of(v[sl])
        full = torch.empty(world * S, dtype=sd, device="cuda")
        u = dict(master=flat[sl], exp_avg=m[sl], exp_avg_sq=v[sl], rank_grads=grads,
                 peer_shards=[None if q == r else peers[q] for q in range(world)], full=full)
        ss.fsdp_step_units([u], r, cfg.fp32_reduce, hp)
        torch.cuda.synchronize()

        def step(lo, hi):
            avg = oracle.grad_average(gs, lo, hi - lo, "bf16", False)
            oracle.adamw16(p0[lo:hi], m0[lo:hi], v0[lo:hi], oracle.to_f32(avg, "bf16"), h, "bf16")

        oracle_chunks(S, step)
        assert_bits_equal(np_of(flat[sl]), p0, "param rank %d" % r)
        assert_bits_equal(np_of(m[sl]), m0, "exp_avg rank %d" % r)
        assert_bits_equal(np_of(v[sl]), v0, "exp_avg_sq rank %d" % r)
        ref = oracle.gather([p0 if q == r else np_of(peers[q]) for q in range(world)], "bf16")
        assert_bits_equal(np_of(full), ref, "full buffer rank %d" % r)
