"""GPU parity of the other pointwise optimizers (SGD, SGD with momentum and
Nesterov, Adamax, Adadelta) on the fused unit step, fsdp_step_units_optim.

Every simulated rank steps its shard three times (t = 1, 2, 3: the first
momentum step and the later ones differ) through the batched unit kernel, with
and without the fused all-gather; the oracle runs the same steps.  Parameter,
state and compute copy must match bit for bit (the bar for fp32 outputs is
1e-6 relative, for 16-bit outputs 1 ulp; the arithmetic is the same operation
sequence, so the result is exact).  State buffers an optimizer does not keep
are never touched.  At full size, every output element of rank 0 is checked.
"""
import numpy as np
import pytest
import torch

import oracle
import sharded_state_amd as ss
from parity import assert_bits_equal, oracle_chunks, assert_bitexact, assert_rel, compare_compute, dt_name, np_of
from workloads import CONFIGS, TORCH_DTYPE, gpt_block, llama_block, moments, param_tensors, rank_grad, scaled

pytestmark = pytest.mark.gpu
H = ss.OptimHP

OPTS = {
    "sgd": H.sgd(lr=1e-2, weight_decay=1e-4),
    "sgd-momentum": H.sgd(lr=1e-2, momentum=0.9, dampening=0.1, weight_decay=1e-4),
    "sgd-nesterov": H.sgd(lr=1e-2, momentum=0.9, nesterov=True),
    "adamax": H.adamax(weight_decay=0.01),
    "adadelta": H.adadelta(weight_decay=0.01),
}


def orc_opt(hp, step):
    """The oracle's hyper-parameters for an OptimHP."""
    if hp.kind == 1:
        return "sgd", oracle.opt("sgd", step=step, lr=hp.lr, weight_decay=hp.weight_decay, momentum=hp.momentum,
                                 dampening=hp.dampening, nesterov=bool(hp.nesterov))
    if hp.kind == 2:
        return "adamax", oracle.opt("adamax", step=step, lr=hp.lr, weight_decay=hp.weight_decay, beta1=hp.beta1,
                                    beta2=hp.beta2, eps=hp.eps)
    return "adadelta", oracle.opt("adadelta", step=step, lr=hp.lr, weight_decay=hp.weight_decay, rho=hp.rho,
                                  eps=hp.eps)


SENTINEL = -12345.5


def _run(cfg, hp, gather, steps=(1, 2, 3)):
    world = cfg.world
    P, Pp, S = ss.fsdp_layout(cfg.numels, world)
    cdt = TORCH_DTYPE[cfg.compute_dt]
    params = [t.cuda() for t in param_tensors(cfg, 0)]
    grads = [rank_grad(cfg, 0, q, Pp).cuda() for q in range(world)]
    m0, v0 = (x.cuda() for x in moments(cfg, 0, 0, Pp, P))
    flat = ss.fsdp_flatten_pad(params, world)
    n = hp.n_states
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    peers = [(torch.randn(S, device="cuda", generator=g) * 0.02).to(cdt) for _ in range(world)]
    kind, _ = orc_opt(hp, 1)
    gs = [np_of(x) for x in grads]
    for r in range(world):
        sl = slice(r * S, (r + 1) * S)
        p, a, b = flat[sl].clone(), m0[sl].clone(), v0[sl].clone()
        if n < 2:
            b.fill_(SENTINEL)
        if n < 1:
            a.fill_(SENTINEL)
        cs = torch.empty(S, dtype=cdt, device="cuda")
        full = torch.empty(world * S, dtype=cdt, device="cuda") if gather else None
        unit = dict(master=p, exp_avg=a, exp_avg_sq=b, rank_grads=grads)
        if gather:
            unit.update(peer_shards=[None if q == r else peers[q] for q in range(world)], full=full,
                        compute_shard=cs)
        else:
            unit.update(compute_shard=cs)
        op, oa, ob = np_of(flat[sl]), np_of(m0[sl]), np_of(v0[sl])
        for t in steps:
            ss.fsdp_step_units([unit], r, cfg.fp32_reduce, hp.at_step(t))
            _, o = orc_opt(hp, t)
            _, oc = oracle.rank_step_opt(kind, gs, r, op, oa, ob, o, dt_name(grads[0].dtype), cfg.fp32_reduce,
                                         cfg.compute_dt)
        torch.cuda.synchronize()
        assert_rel(np_of(p), op, "param rank %d" % r)
        assert_bitexact(np_of(p), op, "param rank %d (bit-exact)" % r)
        if n >= 1:
            assert_bitexact(np_of(a), oa, "state 1 rank %d" % r)
        else:
            assert torch.all(a == SENTINEL), "an unkept state buffer was written"
        if n >= 2:
            assert_bitexact(np_of(b), ob, "state 2 rank %d" % r)
        else:
            assert torch.all(b == SENTINEL), "an unkept state buffer was written"
        compare_compute(np_of(cs), oc, cfg.compute_dt, "compute rank %d" % r)
        assert_bitexact(np_of(cs), oc, "compute rank %d (bit-exact)" % r)
        if gather:
            f = np_of(full)
            assert_bitexact(f[r * S:(r + 1) * S], oc, "own slot rank %d" % r)
            for q in range(world):
                if q != r:
                    assert_bitexact(f[q * S:(q + 1) * S], np_of(peers[q]), "peer slot %d rank %d" % (q, r))


@pytest.mark.parametrize("opt", list(OPTS))
@pytest.mark.parametrize("base,shape,gather", [
    ("gpt2-large-block", gpt_block(64), True),            # N = 2, fp16 grads, fp32 reduce, fp16 compute
    ("gpt3-13b-block", gpt_block(80), False),             # N = 8, shard not 16-byte aligned (scalar path)
    ("llama70b-block", llama_block(64, 80, 224), True),   # N = 8, bf16 grads and reduce, bf16 compute
    ("tiny", [("t", (1001,)), ("u", (7,))], False),        # fp32 everything, ragged tail
])
def test_optimizer_matches_oracle(opt, base, shape, gather):
    print("case", opt, base, gather, flush=True)
    _run(scaled(CONFIGS[base], shape), OPTS[opt], gather)


def test_odd_world_generic_kernel():
    _run(scaled(CONFIGS["gpt3-13b-block"], gpt_block(40), world=3), OPTS["sgd-nesterov"], True)
    _run(scaled(CONFIGS["llama70b-block"], gpt_block(40), world=5), OPTS["adadelta"], False, steps=(1, 2))


def test_batch_of_units_matches_single_units():
    """Several units in one launch give the same bytes as one launch each."""
    cfg = scaled(CONFIGS["gpt2-large-block"], gpt_block(48))
    world = cfg.world
    P, Pp, S = ss.fsdp_layout(cfg.numels, world)
    for hp in (OPTS["sgd-momentum"], OPTS["adamax"]):
        base = []
        for k in range(5):
            grads = [rank_grad(cfg, k, q, Pp).cuda() for q in range(world)]
            flat = ss.fsdp_flatten_pad([t.cuda() for t in param_tensors(cfg, k)], world)
            m, v = (x.cuda() for x in moments(cfg, k, 0, S, P))
            base.append((flat[:S].clone(), m, v, grads))
        one = [[x.clone() if isinstance(x, torch.Tensor) else x for x in b] for b in base]
        many = [[x.clone() if isinstance(x, torch.Tensor) else x for x in b] for b in base]
        outs1 = [torch.empty(S, dtype=torch.float16, device="cuda") for _ in base]
        outsN = [torch.empty(S, dtype=torch.float16, device="cuda") for _ in base]
        for (p, m, v, g), o in zip(one, outs1):
            ss.fsdp_step_units([dict(master=p, exp_avg=m, exp_avg_sq=v, rank_grads=g, compute_shard=o)], 0, True,
                               hp.at_step(2))
        ss.fsdp_step_units([dict(master=p, exp_avg=m, exp_avg_sq=v, rank_grads=g, compute_shard=o)
                            for (p, m, v, g), o in zip(many, outsN)], 0, True, hp.at_step(2))
        torch.cuda.synchronize()
        for (a, b) in zip(one + [outs1], many + [outsN]):
            for x, y in zip(a, b):
                if isinstance(x, torch.Tensor):
                    assert torch.equal(x.view(torch.int16 if x.element_size() == 2 else torch.int32),
                                       y.view(torch.int16 if y.element_size() == 2 else torch.int32))


@pytest.mark.parametrize("opt,name", [("adadelta", "llama70b-block"), ("sgd-nesterov", "gpt3-13b-block"),
                                      ("adamax", "gpt2-xl-model")])
def test_full_size_every_element(opt, name):
    """Rank 0 of the full-size unit with the fused gather, step 2 from the
    workload's state: every element of the parameter and state shards and of
    the full buffer against the oracle (run over disjoint chunks on all host
    threads)."""
    print("case", opt, name, "full size", flush=True)
    cfg = CONFIGS[name]
    hp = OPTS[opt].at_step(2)
    world = cfg.world
    P, Pp, S = ss.fsdp_layout(cfg.numels, world)
    cdt = TORCH_DTYPE[cfg.compute_dt]
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    master = torch.randn(S, device="cuda", generator=g) * 0.02
    m = (torch.randn(S, device="cuda", generator=g) * 1e-4).abs()
    v = (torch.randn(S, device="cuda", generator=g) * 1e-6).abs()
    grads = [rank_grad(cfg, 0, q, Pp, "cuda") for q in range(world)]
    peers = [(torch.randn(S, device="cuda", generator=g) * 0.02).to(cdt) for _ in range(world)]
    gs = [np_of(x[:S]) for x in grads]
    p0, m0, v0 = np_of(master), np_of(m), np_of(v)
    full = torch.empty(world * S, dtype=cdt, device="cuda")
    ss.fsdp_step_units([dict(master=master, exp_avg=m, exp_avg_sq=v, rank_grads=grads, full=full,
                             peer_shards=[None] + peers[1:])], 0, cfg.fp32_reduce, hp)
    torch.cuda.synchronize()
    kind, o = orc_opt(hp, 2)
    comp = np.empty(S, dtype=np.uint16 if cfg.compute_dt != "f32" else np.float32)

    def step(lo, hi):
        avg = oracle.grad_average(gs, lo, hi - lo, cfg.grad_dt, cfg.fp32_reduce)
        g32 = avg if avg.dtype == np.float32 else oracle.to_f32(avg, cfg.grad_dt)
        oracle.opt_step(kind, p0[lo:hi], m0[lo:hi], v0[lo:hi], g32, o)
        comp[lo:hi] = oracle.cast(p0[lo:hi], cfg.compute_dt)

    oracle_chunks(S, step)
    assert_bits_equal(np_of(master), p0, "param")
    if hp.n_states >= 1:
        assert_bits_equal(np_of(m), m0, "state 1")
    if hp.n_states >= 2:
        assert_bits_equal(np_of(v), v0, "state 2")
    ref = oracle.gather([comp] + [np_of(x) for x in peers[1:]], cfg.compute_dt)
    assert_bits_equal(np_of(full), ref, "full buffer")
