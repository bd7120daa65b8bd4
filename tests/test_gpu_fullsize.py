"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times.

At these sizes the oracle checks sampled outputs: the pipeline is pointwise in
the shard element, so the inputs at each sampled position (every rank's
gradient, master, m, v) are copied out before the step and the oracle computes
those outputs one by one.  Samples cover both ends of the shard, the boundary
between the wide and scalar paths, and uniform random positions.  Properties
that hold at any size are checked on the whole buffers on the device: the flat
buffer is the concatenation of the tensors plus +0 padding, the gather is the
concatenation of the shards, and the one-launch unit step gives the same bytes
as the two-call pipeline.
"""
import numpy as np
import pytest
import torch

import oracle
import sharded_state_amd as ss
from parity import assert_bitexact, assert_rel, compare_compute, dt_name, np_of
from workloads import CONFIGS, TORCH_DTYPE, moments, param_tensors, rank_grad

pytestmark = pytest.mark.gpu

NSAMPLE = 200_000


def _bits_equal(a, b):
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def _sample_positions(S, seed):
    rng = np.random.default_rng(seed)
    edge = np.arange(min(S, 4096))
    tail = np.arange(max(0, S - 4096), S)
    mid = (S // 8) * 8
    around = np.arange(max(0, mid - 64), min(S, mid + 64))
    rand = rng.integers(0, S, size=min(NSAMPLE, S))
    return np.unique(np.concatenate([edge, tail, around, rand])).astype(np.int64)


@pytest.mark.parametrize("name", ["tiny", "gpt2-large-block", "gpt2-xl-model", "gpt3-13b-block",
                                  "llama70b-block"])
def test_full_size_unit(name):
    cfg = CONFIGS[name]
    print("case", name, "full size", flush=True)
    dev = "cuda"
    world = cfg.world
    P, Pp, S = ss.fsdp_layout(cfg.numels, world)
    cdt = TORCH_DTYPE[cfg.compute_dt]
    hp = ss.AdamWHP(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.step)

    # flatten + pad (bench's init step); property: concatenation + zero tail
    params = param_tensors(cfg, 0, dev)
    flat = ss.fsdp_flatten_pad(params, world)
    cat = torch.cat([t.reshape(-1) for t in params])
    assert flat.numel() == Pp and _bits_equal(flat[:P], cat)
    assert torch.count_nonzero(flat[P:].view(torch.int32)) == 0
    del cat
    views = ss.fsdp_unflatten_views(flat, cfg.shapes)
    for v, t in zip(views, params):
        assert _bits_equal(v, t)
    offs = oracle.offsets(cfg.numels)
    assert [v.data_ptr() - flat.data_ptr() for v in views] == [4 * int(o) for o in offs]
    del params, views

    grads = [rank_grad(cfg, 0, q, Pp, dev) for q in range(world)]
    m, v = moments(cfg, 0, 0, Pp, P, dev)
    master = flat
    ranks = sorted({0, world - 1})
    samples = {}
    for r in ranks:
        idx = _sample_positions(S, r)
        pos = torch.from_numpy(r * S + idx).to(dev)
        samples[r] = (idx, [np_of(g[pos]) for g in grads], np_of(master[pos]), np_of(m[pos]), np_of(v[pos]))
    keep0 = (master[:S].clone(), m[:S].clone(), v[:S].clone())

    # two-call pipeline for every rank, as the gather needs every shard
    compute = [torch.empty(S, dtype=cdt, device=dev) for _ in range(world)]
    gshard0 = ss.fsdp_reduce_scatter_local(grads, 0, cfg.fp32_reduce, shard_numel=S)
    for r in range(world):
        sl = slice(r * S, (r + 1) * S)
        ss.fsdp_sharded_adamw(master[sl], m[sl], v[sl], grads, r, cfg.fp32_reduce, hp, compute_shard=compute[r])
    full = ss.fsdp_unshard_gather(compute)
    torch.cuda.synchronize()
    for q in range(world):
        assert _bits_equal(full[q * S:(q + 1) * S], compute[q])

    h = oracle.hp(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.step)
    gd = dt_name(grads[0].dtype)
    for r in ranks:
        idx, gs, p0, m0, v0 = samples[r]
        sel = torch.from_numpy(idx).to(dev)
        p, mm, vv = p0.copy(), m0.copy(), v0.copy()
        avg, comp = oracle.elementwise_step(gs, p, mm, vv, h, gd, cfg.fp32_reduce, cfg.compute_dt)
        sl = slice(r * S, (r + 1) * S)
        for nm, got, ref in (("master", master[sl][sel], p), ("exp_avg", m[sl][sel], mm),
                             ("exp_avg_sq", v[sl][sel], vv)):
            g_ = np_of(got)
            assert_rel(g_, ref, "%s rank %d" % (nm, r))
            assert_bitexact(g_, ref, "%s rank %d (bit-exact)" % (nm, r))
        compare_compute(np_of(compute[r][sel]), comp, cfg.compute_dt, "compute rank %d" % r)
        compare_compute(np_of(full[r * S:(r + 1) * S][sel]), comp, cfg.compute_dt, "full rank %d" % r)
        if r == 0:
            assert_bitexact(np_of(gshard0[sel]), avg, "reduce-scatter rank 0")

    # the one-launch unit step for rank 0 from the same initial state
    p0, m0, v0 = keep0
    full2 = torch.empty(world * S, dtype=cdt, device=dev)
    persistent = torch.empty(S, dtype=cdt, device=dev) if cfg.gathers > 1 else None
    peers = [None] + compute[1:]
    ss.fsdp_step_unit(p0, m0, v0, grads, 0, cfg.fp32_reduce, hp, peers, full2, compute_shard=persistent)
    if cfg.gathers > 1:   # reshard after forward: gather again before backward
        full3 = ss.fsdp_unshard_gather([persistent] + compute[1:])
    torch.cuda.synchronize()
    assert _bits_equal(p0, master[:S]) and _bits_equal(m0, m[:S]) and _bits_equal(v0, v[:S])
    assert _bits_equal(full2, full)
    if cfg.gathers > 1:
        assert _bits_equal(persistent, compute[0]) and _bits_equal(full3, full)


def test_sharded_state_is_one_nth_of_unsharded_state():
    """The per-worker memory invariant every page agrees on, measured with the
    allocator: one rank's persistent state (fp32 master, m, v; compute shard;
    fp32 gradient shard) is 1/N of the unsharded unit's (world = 1), plus the
    padding, and matches the oracle's closed form."""
    cfg = CONFIGS["gpt2-large-block"]
    per_elt = 12 + 2 + 4
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    full = ss.RankState(cfg.numels, 1, 0, torch.float16, torch.float32)
    unsharded = torch.cuda.memory_allocated() - base
    assert sum(full.nbytes().values()) == full.numel * per_elt
    assert 0 <= unsharded - full.numel * per_elt <= 5 * (2 << 20)
    del full
    for world in (2, 7, 8):
        base = torch.cuda.memory_allocated()
        st = ss.RankState(cfg.numels, world, world - 1, torch.float16, torch.float32)
        sharded = torch.cuda.memory_allocated() - base
        pad = st.padded_numel - st.numel
        exact = sum(st.nbytes().values())
        # exact accounting: N shards hold the unsharded bytes plus the padding
        assert exact == st.shard_numel * per_elt
        assert world * exact == st.numel * per_elt + pad * per_elt
        assert exact == oracle.memory_per_worker(cfg.numel, world, 1, 1, 1, 2, 4, 12).sum()
        # measured: large blocks are rounded up to 2 MiB by torch's caching allocator
        slack = 5 * (2 << 20)
        assert 0 <= sharded - exact <= slack
        assert abs(world * sharded - unsharded) <= world * slack + pad * per_elt
        del st


@pytest.mark.parametrize("name,per_launch", [("gpt2-large-block", 36), ("gpt3-13b-block", 4),
                                             ("llama70b-block", 2)])
def test_full_size_batched_launch(name, per_launch):
    """The benchmark's call: `per_launch` distinct full-size units of rank 0 in
    one fsdp_step_units call with the gather (packed into launches as the
    library packs them; and,
    with two gathers per step, the persistent own shard).  Per unit: sampled
    master, m, v and own-slot values against the oracle; the peer slots equal
    the peer shards bit for bit."""
    cfg = CONFIGS[name]
    print("case", name, per_launch, "units per launch", flush=True)
    dev = "cuda"
    world = cfg.world
    P, Pp, S = ss.fsdp_layout(cfg.numels, world)
    cdt = TORCH_DTYPE[cfg.compute_dt]
    hp = ss.AdamWHP(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.step)
    h = oracle.hp(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.step)
    gd = cfg.grad_dt
    units, refs = [], []
    for b in range(per_launch):
        flat = ss.fsdp_flatten_pad(param_tensors(cfg, b, dev), world)
        master = flat[:S].clone()
        del flat
        grads = [rank_grad(cfg, b, q, Pp, dev) for q in range(world)]
        m, v = moments(cfg, b, 0, S, P, dev)
        g = torch.Generator(device=dev)
        g.manual_seed(100 + b)
        peers = [None] + [(torch.randn(S, device=dev, generator=g) * 0.02).to(cdt) for _ in range(world - 1)]
        full = torch.empty(world * S, dtype=cdt, device=dev)
        persistent = torch.empty(S, dtype=cdt, device=dev) if cfg.gathers > 1 else None
        rng = np.random.default_rng(b)
        idx = np.unique(np.concatenate([np.arange(1024), np.arange(S - 1024, S), rng.integers(0, S, 20_000)]))
        sel = torch.from_numpy(idx).to(dev)
        refs.append((idx, sel, [np_of(x[sel]) for x in grads], np_of(master[sel]), np_of(m[sel]), np_of(v[sel])))
        units.append(dict(master=master, exp_avg=m, exp_avg_sq=v, rank_grads=grads, peer_shards=peers, full=full,
                          compute_shard=persistent))
    ss.fsdp_step_units(units, 0, cfg.fp32_reduce, hp)
    torch.cuda.synchronize()
    for b, (u, (idx, sel, gs, p0, m0, v0)) in enumerate(zip(units, refs)):
        p, mm, vv = p0.copy(), m0.copy(), v0.copy()
        _, comp = oracle.elementwise_step(gs, p, mm, vv, h, gd, cfg.fp32_reduce, cfg.compute_dt)
        assert_bitexact(np_of(u["master"][sel]), p, "master, unit %d" % b)
        assert_bitexact(np_of(u["exp_avg"][sel]), mm, "exp_avg, unit %d" % b)
        assert_bitexact(np_of(u["exp_avg_sq"][sel]), vv, "exp_avg_sq, unit %d" % b)
        own = u["full"][:S]
        assert_bitexact(np_of(own[sel]), comp, "own slot, unit %d" % b)
        if u["compute_shard"] is not None:
            assert _bits_equal(u["compute_shard"], own)
        for q in range(1, world):
            assert _bits_equal(u["full"][q * S:(q + 1) * S], u["peer_shards"][q]), (b, q)
