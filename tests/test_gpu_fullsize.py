"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times, on every element.

Each case builds a workload's pool of distinct units at full size for one
simulated rank -- rank 0 and rank N-1 -- and steps them with one
fsdp_step_units call, which the library packs into launches exactly as the
benchmark's calls are packed: GPT-2 Large's 36 blocks six to a launch with
the peers' copies in a launch of their own, the GPT-2 XL shard and the 70B
blocks in 2^26-element slices, the 13B blocks one per launch with the
persistent own copy and a second all-gather.  Then every element of the
rank's outputs is compared with the oracle run on the same input bytes over
disjoint chunks on all host threads (checker side only):
  * the standalone reduce-scatter shard: bit-exact;
  * master, m, v: bit-exact (which meets max relative error <= 1e-6);
  * the whole full buffer (own slot and every peer slot) against the oracle's
    gather of the oracle's compute shard and the peers' shards: <= 1 ulp
    (16-bit) / rel 1e-6 (fp32) on the own slot, bit-exact elsewhere (in
    practice bit-exact everywhere);
  * with two gathers: the persistent own copy and the second gather.
Flatten + pad of the first unit is compared with the oracle's flatten on
every element too, and the per-tensor views with the oracle's unflatten
offsets.

The pages' claim behind the oracle: sharded results equal the unsharded
(DDP) step element for element ("Fully Sharded Data Parallel: faster AI
training with fewer GPUs", end of "From all-reduce to sharded parameters").
"""
import numpy as np
import pytest
import torch

import oracle
import sharded_state_amd as ss
from parity import assert_bits_equal, assert_compute_close, dt_name, np_of, oracle_rank_step_threaded
from workloads import CONFIGS, TORCH_DTYPE, moments, param_tensors, rank_grads

pytestmark = pytest.mark.gpu

# (workload, distinct units stepped in one call): the benchmark's pools
CASES = [("tiny", 1), ("gpt2-large-block", 36), ("gpt2-xl-model", 1), ("gpt3-13b-block", 4),
         ("llama70b-block", 2)]


def _bits_equal(a, b):
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def _check_flatten(cfg, flat, params):
    """Every element of the device flat buffer against the oracle's flatten of
    the same host tensors; views at the oracle's offsets."""
    P, Pp, _ = ss.fsdp_layout(cfg.numels, cfg.world)
    host = [np_of(t).reshape(-1) for t in params]
    assert_bits_equal(np_of(flat), oracle.flatten_pad(host, cfg.world, "f32"), "flatten + pad")
    del host
    views = ss.fsdp_unflatten_views(flat, cfg.shapes)
    offs = oracle.offsets(cfg.numels)
    assert [v.data_ptr() - flat.data_ptr() for v in views] == [4 * int(o) for o in offs]
    for v, t in zip(views, params):
        assert tuple(v.shape) == tuple(t.shape) and _bits_equal(v, t)


@pytest.mark.parametrize("end", ["first", "last"])
@pytest.mark.parametrize("name,blocks", CASES)
def test_full_size_every_element(name, blocks, end):
    cfg = CONFIGS[name]
    dev = "cuda"
    world = cfg.world
    rank = 0 if end == "first" else world - 1
    print("case %s x%d units, rank %d of %d, full size, every element" % (name, blocks, rank, world), flush=True)
    P, Pp, S = ss.fsdp_layout(cfg.numels, world)
    sl = slice(rank * S, (rank + 1) * S)
    cdt = cfg.compute_dt
    cdt_t = TORCH_DTYPE[cdt]
    hp = ss.AdamWHP(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.step)
    h = oracle.hp(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.step)

    units, hosts, gshards = [], [], []
    for b in range(blocks):
        params = param_tensors(cfg, b, dev)
        flat = ss.fsdp_flatten_pad(params, world)
        if b == 0 and rank == 0:
            _check_flatten(cfg, flat, params)
        del params
        master = flat[sl].clone()
        del flat
        grads = list(rank_grads(cfg, b, Pp, dev).unbind(0))   # the benchmark's buffers: rows of one allocation
        m, v = moments(cfg, b, rank * S, S, P, dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(100 + 10 * b + rank)
        peers = [None if q == rank else (torch.randn(S, device=dev, generator=gen) * 0.02).to(cdt_t)
                 for q in range(world)]
        full = torch.empty(world * S, dtype=cdt_t, device=dev)
        persistent = torch.empty(S, dtype=cdt_t, device=dev) if cfg.gathers > 1 else None
        hosts.append(dict(grads=[np_of(g[sl]) for g in grads], p=np_of(master), m=np_of(m), v=np_of(v),
                          peers=[None if x is None else np_of(x) for x in peers]))
        gshards.append(ss.fsdp_reduce_scatter_local(grads, rank, cfg.fp32_reduce, shard_numel=S))
        units.append(dict(master=master, exp_avg=m, exp_avg_sq=v, rank_grads=grads, peer_shards=peers, full=full,
                          compute_shard=persistent))
    print("  inputs ready; stepping %d units in one call" % blocks, flush=True)
    ss.fsdp_step_units(units, rank, cfg.fp32_reduce, hp)
    second = []
    if cfg.gathers > 1:   # reshard after forward: gather again, from the persistent own copy
        for u in units:
            second.append(ss.fsdp_unshard_gather([u["compute_shard"] if q == rank else u["peer_shards"][q]
                                                  for q in range(world)]))
    torch.cuda.synchronize()
    gd = dt_name(units[0]["rank_grads"][0].dtype)
    for b, (u, hst) in enumerate(zip(units, hosts)):
        p, m, v = hst["p"], hst["m"], hst["v"]
        avg, comp = oracle_rank_step_threaded(hst["grads"], p, m, v, h, gd, cfg.fp32_reduce, cdt)
        assert_bits_equal(np_of(gshards[b]), avg, "reduce-scatter, unit %d" % b)
        assert_bits_equal(np_of(u["master"]), p, "master, unit %d" % b)
        assert_bits_equal(np_of(u["exp_avg"]), m, "exp_avg, unit %d" % b)
        assert_bits_equal(np_of(u["exp_avg_sq"]), v, "exp_avg_sq, unit %d" % b)
        shards = [comp if q == rank else hst["peers"][q] for q in range(world)]
        ref_full = oracle.gather(shards, cdt)
        got_full = np_of(u["full"])
        assert_compute_close(got_full[sl], comp, cdt, "own slot, unit %d" % b)
        for q in range(world):
            if q != rank:
                assert_bits_equal(got_full[q * S:(q + 1) * S], ref_full[q * S:(q + 1) * S],
                                  "peer slot %d, unit %d" % (q, b))
        if cfg.gathers > 1:
            assert_compute_close(np_of(u["compute_shard"]), comp, cdt, "persistent own copy, unit %d" % b)
            assert_compute_close(np_of(second[b]), ref_full, cdt, "second gather, unit %d" % b)
        del got_full, ref_full, shards, avg, comp
        hosts[b] = None
    print("  every element of %d units matches" % blocks, flush=True)


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
