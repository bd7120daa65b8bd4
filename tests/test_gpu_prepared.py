"""GPU tests of the prepared calls (prepare_step_units, prepare_offload_step_units):
one marshalled call re-issued over several training steps must take each
step's t -- AdamW's bias corrections 1 - beta1^t and 1 - beta2^t, SGD's first
momentum step -- and run on the stream it is issued on.  Each step is compared
bit for bit with the oracle at the same t.
"""
import numpy as np
import pytest
import torch

import oracle
import sharded_state_amd as ss
from parity import assert_bitexact, np_of
from workloads import CONFIGS, gpt_block, moments, param_tensors, rank_grad, scaled

pytestmark = pytest.mark.gpu


def _unit(cfg, rank, dev="cuda"):
    P, Pp, S = ss.fsdp_layout(cfg.numels, cfg.world)
    flat = ss.fsdp_flatten_pad([t.to(dev) for t in param_tensors(cfg, 0)], cfg.world)
    sl = slice(rank * S, (rank + 1) * S)
    m, v = (x.to(dev) for x in moments(cfg, 0, 0, Pp, P))
    grads = [rank_grad(cfg, 0, q, Pp).to(dev) for q in range(cfg.world)]
    return S, flat[sl].clone(), m[sl].clone(), v[sl].clone(), grads


def test_prepared_adamw_call_takes_each_step():
    cfg = scaled(CONFIGS["gpt2-large-block"], gpt_block(64) + [("odd", (5,))], mv_sigma=1e-4)
    rank = 1
    print("case prepared AdamW, N=%d rank %d" % (cfg.world, rank), flush=True)
    S, p, m, v, grads = _unit(cfg, rank)
    cdt = torch.float16
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    peers = [(torch.randn(S, device="cuda", generator=g) * 0.02).to(cdt) if q != rank else None
             for q in range(cfg.world)]
    full = torch.empty(cfg.world * S, dtype=cdt, device="cuda")
    op, om, ov = np_of(p), np_of(m), np_of(v)
    og = oracle.reduce_scatter([np_of(x) for x in grads], rank, cfg.grad_dt, cfg.fp32_reduce)
    hp = ss.AdamWHP(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, 1)
    call = ss.prepare_step_units([dict(master=p, exp_avg=m, exp_avg_sq=v, rank_grads=grads, peer_shards=peers,
                                       full=full)], rank, cfg.fp32_reduce, hp)
    hp.step = 99                  # the call keeps its own copy: the caller's struct is not read
    side = torch.cuda.Stream()
    for t in (1, 2, 3, 10):
        if t == 3:
            side.wait_stream(torch.cuda.current_stream())
            call(step=t, stream=side)          # an explicit stream
            torch.cuda.current_stream().wait_stream(side)
        elif t == 10:
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):      # the current stream at the time of the call
                call(step=t)
            torch.cuda.current_stream().wait_stream(side)
        else:
            call(step=t)
        assert call.hp.step == t
        torch.cuda.synchronize()
        oracle.adamw(op, om, ov, og, oracle.hp(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, t))
        assert_bitexact(np_of(p), op, "master t=%d" % t)
        assert_bitexact(np_of(m), om, "exp_avg t=%d" % t)
        assert_bitexact(np_of(v), ov, "exp_avg_sq t=%d" % t)
        assert_bitexact(np_of(full[rank * S:(rank + 1) * S]), oracle.cast(op, "f16"), "own slot t=%d" % t)
    with pytest.raises(ValueError):
        call(step=0)


def test_prepared_sgd_momentum_call_starts_its_buffer_once():
    """SGD with momentum copies the gradient into the buffer at t = 1 only."""
    cfg = scaled(CONFIGS["gpt2-large-block"], gpt_block(48))
    print("case prepared SGD momentum", flush=True)
    S, p, buf, _, grads = _unit(cfg, 0)
    buf.fill_(123.0)              # must be ignored at t = 1
    comp = torch.empty(S, dtype=torch.float16, device="cuda")
    o = ss.OptimHP.sgd(lr=1e-2, momentum=0.9, dampening=0.1, weight_decay=1e-4)
    call = ss.prepare_step_units([dict(master=p, exp_avg=buf, rank_grads=grads, compute_shard=comp)], 0,
                                 cfg.fp32_reduce, o)
    op, ob = np_of(p), np_of(buf)
    og = oracle.reduce_scatter([np_of(x) for x in grads], 0, cfg.grad_dt, cfg.fp32_reduce)
    for t in (1, 2, 3):
        call(step=t)
        torch.cuda.synchronize()
        oracle.sgd(op, ob, og, oracle.opt("sgd", step=t, lr=1e-2, momentum=0.9, dampening=0.1, weight_decay=1e-4))
        assert_bitexact(np_of(p), op, "master t=%d" % t)
        assert_bitexact(np_of(buf), ob, "momentum buffer t=%d" % t)
        assert_bitexact(np_of(comp), oracle.cast(op, "f16"), "compute t=%d" % t)


def test_prepared_offload_call_takes_each_step():
    cfg = scaled(CONFIGS["llama70b-block"], gpt_block(40))
    rank = cfg.world - 1
    print("case prepared offload, N=%d rank %d" % (cfg.world, rank), flush=True)
    S, p, m, v, grads = _unit(cfg, rank)
    st = ss.OffloadState(p, grads[0].dtype, cfg.fp32_reduce, torch.bfloat16, "cuda", exp_avg=m, exp_avg_sq=v)
    comp = torch.empty(S, dtype=torch.bfloat16, device="cuda")
    call = ss.prepare_offload_step_units([(st, grads, comp)], rank, cfg.fp32_reduce, ss.AdamWHP(), chunk_numel=1000,
                                         n_threads=3)
    op, om, ov = np_of(p), np_of(m), np_of(v)
    og = oracle.to_f32(oracle.reduce_scatter([np_of(x) for x in grads], rank, cfg.grad_dt, cfg.fp32_reduce), "bf16")
    for t in (1, 2, 5):
        call(step=t)
        torch.cuda.synchronize()
        oracle.adamw(op, om, ov, og, oracle.hp(step=t))
        assert_bitexact(np_of(st.master), op, "offload master t=%d" % t)
        assert_bitexact(np_of(st.exp_avg), om, "offload exp_avg t=%d" % t)
        assert_bitexact(np_of(st.exp_avg_sq), ov, "offload exp_avg_sq t=%d" % t)
        assert np.array_equal(np_of(comp), oracle.cast(op, "bf16")), t


def test_unit_config_step_is_the_flags_step():
    """UnitConfig.step with fairseq's --fp16 --fp32-reduce-scatter (reshard after
    forward: two gathers, a persistent compute shard) steps the unit as the
    flags say: fp16 gradients reduced in fp32, fp32 master, fp16 compute copy
    in the own slot and in the persistent shard, the peer's slot copied."""
    cfg = scaled(CONFIGS["gpt3-13b-block"], gpt_block(64) + [("odd", (3,))], world=2)
    rank = 1
    c = ss.from_fairseq(cfg.world, rank, fp16=True, fp32_reduce_scatter=True)
    print("case UnitConfig step, N=%d rank %d" % (cfg.world, rank), flush=True)
    S, p, m, v, grads = _unit(cfg, rank)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    peers = [(torch.randn(S, device="cuda", generator=g) * 0.02).half() if q != rank else None
             for q in range(cfg.world)]
    full = torch.empty(cfg.world * S, dtype=torch.float16, device="cuda")
    comp = torch.empty(S, dtype=torch.float16, device="cuda")
    op, om, ov = np_of(p), np_of(m), np_of(v)
    og = oracle.reduce_scatter([np_of(x) for x in grads], rank, "f16", True)
    c.step([dict(master=p, exp_avg=m, exp_avg_sq=v, rank_grads=grads, peer_shards=peers, full=full,
                 compute_shard=comp)], ss.AdamWHP(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, 1))
    torch.cuda.synchronize()
    oracle.adamw(op, om, ov, og, oracle.hp(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, 1))
    assert_bitexact(np_of(p), op, "master")
    assert_bitexact(np_of(m), om, "exp_avg")
    assert_bitexact(np_of(v), ov, "exp_avg_sq")
    own = oracle.cast(op, "f16")
    assert_bitexact(np_of(full[rank * S:(rank + 1) * S]), own, "own slot")
    assert_bitexact(np_of(comp), own, "persistent compute shard")
    assert_bitexact(np_of(full[:S]), np_of(peers[0]), "peer slot")
    with pytest.raises(ValueError, match="persistent"):
        c.step([dict(master=p, exp_avg=m, exp_avg_sq=v, rank_grads=grads, peer_shards=peers, full=full)],
               ss.AdamWHP())
