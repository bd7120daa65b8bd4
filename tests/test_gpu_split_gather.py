"""GPU: the two forms of the unit step's all-gather give the same bytes.

A step launch with a gather copies the peers' shards in its own trip, or -- for
an optimizer that keeps state and at least 2^24 shard elements in the launch,
with fp32 or 16-bit state (unit_gather_split) -- writes only the own slots and
leaves the copies to a batched copy launch.  Here the same units are stepped once as one
batch (past the threshold: two launches) and once one unit per call (under it:
the fused form), from identical inputs, and every output is compared bit for
bit; the full buffers are also checked against the concatenation of the own
compute shard and the peers' shards.
"""
import pytest
import torch

import sharded_state_amd as ss
from parity import np_of

pytestmark = pytest.mark.gpu

SPLIT_ELEMS = 1 << 24


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _units(world, rank, sizes, gdt, cdt, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = []
    for S in sizes:
        grads = [(torch.randn(world * S, device="cuda", generator=g) * 1e-3).to(gdt) for _ in range(world)]
        master = torch.randn(S, device="cuda", generator=g) * 0.02
        m = torch.randn(S, device="cuda", generator=g) * 1e-3
        v = torch.rand(S, device="cuda", generator=g) * 1e-6
        peers = [None if q == rank else (torch.randn(S, device="cuda", generator=g) * 0.02).to(cdt)
                 for q in range(world)]
        out.append(dict(master=master, exp_avg=m, exp_avg_sq=v, rank_grads=grads, peer_shards=peers,
                        full=torch.full((world * S,), float("nan"), dtype=cdt, device="cuda")))
    return out


def _clone(units):
    return [dict(master=u["master"].clone(), exp_avg=u["exp_avg"].clone(), exp_avg_sq=u["exp_avg_sq"].clone(),
                 rank_grads=u["rank_grads"], peer_shards=u["peer_shards"],
                 full=torch.full_like(u["full"], float("nan"))) for u in units]


HPS = {
    "adamw": lambda: ss.AdamWHP(1e-3, 0.9, 0.999, 1e-8, 0.01, 3),
    "adamax": lambda: ss.OptimHP.adamax(weight_decay=0.01, step=3),
    "adadelta": lambda: ss.OptimHP.adadelta(weight_decay=0.01, step=3),
    "sgd-momentum": lambda: ss.OptimHP.sgd(lr=1e-2, momentum=0.9, weight_decay=1e-4, step=3),
    "sgd": lambda: ss.OptimHP.sgd(lr=1e-2, weight_decay=1e-4, step=3),
}


@pytest.mark.parametrize("world,gdt,fp32_reduce,cdt,opt", [
    (2, torch.float16, True, torch.float16, "adamw"),
    (2, torch.bfloat16, False, torch.bfloat16, "adamax"),
    (2, torch.float16, True, torch.float32, "adadelta"),
    (2, torch.float16, True, torch.float16, "sgd-momentum"),
    (2, torch.float16, True, torch.float16, "sgd"),
    (8, torch.bfloat16, False, torch.bfloat16, "adamw"),
    (4, torch.float32, True, torch.float16, "adamw"),
])
def test_batched_split_gather_equals_fused(world, gdt, fp32_reduce, cdt, opt):
    hp = HPS[opt]()
    n_states = hp.n_states if isinstance(hp, ss.OptimHP) else 2
    # three units, each under the threshold, together over it; ragged sizes
    sizes = [(SPLIT_ELEMS // 2) + 8 * 37 + 5, (SPLIT_ELEMS // 3) + 1, (SPLIT_ELEMS // 4) + 512]
    print("case", world, gdt, fp32_reduce, cdt, opt, sizes, flush=True)
    assert all(not ss.unit_gather_split(torch.float32, n_states, S) for S in sizes)
    split = ss.unit_gather_split(torch.float32, n_states, sum(sizes))
    assert split == (n_states >= 1)
    rank = world - 1
    a = _units(world, rank, sizes, gdt, cdt, 7)
    b = _clone(a)
    ss.fsdp_step_units(a, rank, fp32_reduce, hp)                 # one launch table: split when n_states >= 1
    for u in b:
        ss.fsdp_step_units([u], rank, fp32_reduce, hp)           # one unit per call: the fused form
    torch.cuda.synchronize()
    for k, (ua, ub, S) in enumerate(zip(a, b, sizes)):
        for key in ("master", "exp_avg", "exp_avg_sq", "full"):
            if key == "exp_avg" and n_states < 1 or key == "exp_avg_sq" and n_states < 2:
                continue
            assert torch.equal(_bits(ua[key]), _bits(ub[key])), (k, key)
        full = ua["full"]
        own = ua["master"].to(cdt) if cdt != torch.float32 else ua["master"]
        assert torch.equal(_bits(full[rank * S:(rank + 1) * S]), _bits(own)), k
        for q in range(world):
            if q != rank:
                assert torch.equal(_bits(full[q * S:(q + 1) * S]), _bits(ua["peer_shards"][q])), (k, q)


@pytest.mark.parametrize("world,state", [(2, torch.bfloat16), (8, torch.bfloat16), (4, torch.float16)])
def test_sixteen_bit_state_split_gather_equals_fused(world, state):
    """16-bit parameter, m and v (the parameter shard is the compute shard):
    three units under the 2^24-element threshold stepped one per call (the
    fused form) and together (over it: the step, then the batched copies) give
    the same bits in every output, and the full buffer holds the new parameter
    shard in its own slot and the peers' shards in theirs."""
    sizes = [(SPLIT_ELEMS // 2) + 8 * 37 + 5, (SPLIT_ELEMS // 3) + 1, (SPLIT_ELEMS // 4) + 512]
    print("case", world, state, sizes, flush=True)
    assert all(not ss.unit_gather_split(state, 2, S) for S in sizes)
    assert ss.unit_gather_split(state, 2, sum(sizes))
    rank = 1
    hp = ss.AdamWHP(1e-3, 0.9, 0.999, 1e-8, 0.01, 3)
    gdt = torch.bfloat16 if state == torch.bfloat16 else torch.float16
    a = _units(world, rank, sizes, gdt, state, 17)
    for u in a:
        for key in ("master", "exp_avg", "exp_avg_sq"):
            u[key] = u[key].to(state)
    b = _clone(a)
    ss.fsdp_step_units(a, rank, False, hp)
    for u in b:
        ss.fsdp_step_units([u], rank, False, hp)
    torch.cuda.synchronize()
    for k, (ua, ub, S) in enumerate(zip(a, b, sizes)):
        for key in ("master", "exp_avg", "exp_avg_sq", "full"):
            assert torch.equal(_bits(ua[key]), _bits(ub[key])), (k, key)
        full = ua["full"]
        assert torch.equal(_bits(full[rank * S:(rank + 1) * S]), _bits(ua["master"])), k
        for q in range(world):
            if q != rank:
                assert torch.equal(_bits(full[q * S:(q + 1) * S]), _bits(ua["peer_shards"][q])), (k, q)


def test_split_gather_generic_world_one_unit_per_launch():
    """World 3 takes the generic kernel, one unit per launch: a unit of 2^24
    shard elements takes the split form and matches the two-call pipeline
    (reduce-scatter + step without gather, then the all-gather)."""
    world, S, rank = 3, SPLIT_ELEMS, 1
    assert ss.unit_gather_split(torch.float32, 2, S)
    hp = ss.AdamWHP(1e-3, 0.9, 0.999, 1e-8, 0.01, 2)
    a = _units(world, rank, [S], torch.float16, torch.bfloat16, 11)
    b = _clone(a)
    ss.fsdp_step_units(a, rank, True, hp)
    u = b[0]
    comp = torch.empty(S, dtype=torch.bfloat16, device="cuda")
    ss.fsdp_step_units([dict(master=u["master"], exp_avg=u["exp_avg"], exp_avg_sq=u["exp_avg_sq"],
                             rank_grads=u["rank_grads"], compute_shard=comp)], rank, True, hp)
    shards = [comp if q == rank else u["peer_shards"][q] for q in range(world)]
    full = ss.fsdp_unshard_gather(shards)
    torch.cuda.synchronize()
    for key in ("master", "exp_avg", "exp_avg_sq"):
        assert torch.equal(_bits(a[0][key]), _bits(u[key])), key
    assert torch.equal(_bits(a[0]["full"]), _bits(full))
    assert np_of(comp).size == S


def test_one_call_with_a_split_launch_and_a_fused_launch():
    """45 units at N = 2 take two launches (40 + 5): the first holds 2^24+ shard
    elements and splits, the second does not; every unit still matches its
    one-unit (fused) step bit for bit."""
    world, rank, S, n = 2, 0, 420_000, 45
    assert ss.unit_gather_split(torch.float32, 2, 40 * S) and not ss.unit_gather_split(torch.float32, 2, 5 * S)
    hp = ss.AdamWHP(1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    a = _units(world, rank, [S + 8 * (k % 3) for k in range(n)], torch.float16, torch.float16, 21)
    b = _clone(a)
    ss.fsdp_step_units(a, rank, True, hp)
    for u in b:
        ss.fsdp_step_units([u], rank, True, hp)
    torch.cuda.synchronize()
    for k, (ua, ub) in enumerate(zip(a, b)):
        for key in ("master", "exp_avg", "exp_avg_sq", "full"):
            assert torch.equal(_bits(ua[key]), _bits(ub[key])), (k, key)


def test_unit_above_the_launch_cap_is_stepped_in_slices():
    """A shard of 2^26 + 1003 elements is stepped as a 2^26-element slice and a
    ragged remainder, each a launch (with its peers' copies); every element of
    master, m, v and the full buffer matches the oracle bit for bit."""
    import numpy as np
    import oracle
    from parity import assert_bits_equal, oracle_rank_step_threaded
    world, rank = 2, 0
    S = (1 << 26) + 1003
    assert ss.units_in_launch(world, [S]) == (1, 1 << 26)
    u = _units(world, rank, [S], torch.float16, torch.float16, 31)[0]
    gs = [np_of(g[:S]) for g in u["rank_grads"]]              # rank 0's block is the first S elements
    p, m, v = (np_of(u[k]) for k in ("master", "exp_avg", "exp_avg_sq"))
    h = oracle.hp(1e-3, 0.9, 0.999, 1e-8, 0.01, 2)
    ss.fsdp_step_units([u], rank, True, ss.AdamWHP(1e-3, 0.9, 0.999, 1e-8, 0.01, 2))
    torch.cuda.synchronize()
    _, comp = oracle_rank_step_threaded(gs, p, m, v, h, "f16", True, "f16")
    assert_bits_equal(np_of(u["master"]), p, "master")
    assert_bits_equal(np_of(u["exp_avg"]), m, "exp_avg")
    assert_bits_equal(np_of(u["exp_avg_sq"]), v, "exp_avg_sq")
    assert_bits_equal(np_of(u["full"]), np.concatenate([comp, np_of(u["peer_shards"][1])]), "full buffer")


def test_sixteen_bit_state_unit_above_the_launch_cap():
    """The same slicing with bf16 parameter, m and v (the peers' copies in a
    launch after each slice): every element matches the oracle's 16-bit AdamW
    bit for bit."""
    import numpy as np
    import oracle
    from parity import assert_bits_equal, oracle_chunks
    world, rank = 2, 1
    S = (1 << 26) + 517
    g = torch.Generator(device="cuda")
    g.manual_seed(41)
    bf = torch.bfloat16
    grads = [(torch.randn(world * S, device="cuda", generator=g) * 1e-3).half() for _ in range(world)]
    u = dict(master=(torch.randn(S, device="cuda", generator=g) * 0.02).to(bf),
             exp_avg=(torch.randn(S, device="cuda", generator=g) * 1e-3).to(bf),
             exp_avg_sq=(torch.rand(S, device="cuda", generator=g) * 1e-6).to(bf), rank_grads=grads,
             peer_shards=[(torch.randn(S, device="cuda", generator=g) * 0.02).to(bf), None],
             full=torch.empty(world * S, dtype=bf, device="cuda"))
    gs = [np_of(x[rank * S:(rank + 1) * S]) for x in grads]
    p, m, v = (np_of(u[k]) for k in ("master", "exp_avg", "exp_avg_sq"))
    ss.fsdp_step_units([u], rank, True, ss.AdamWHP(1e-3, 0.9, 0.999, 1e-8, 0.01, 3))
    torch.cuda.synchronize()
    h = oracle.hp(1e-3, 0.9, 0.999, 1e-8, 0.01, 3)

    def step(lo, hi):
        avg = oracle.grad_average(gs, lo, hi - lo, "f16", True)
        oracle.adamw16(p[lo:hi], m[lo:hi], v[lo:hi], avg, h, "bf16")

    oracle_chunks(S, step)
    assert_bits_equal(np_of(u["master"]), p, "parameter")
    assert_bits_equal(np_of(u["exp_avg"]), m, "exp_avg")
    assert_bits_equal(np_of(u["exp_avg_sq"]), v, "exp_avg_sq")
    assert_bits_equal(np_of(u["full"]), np.concatenate([np_of(u["peer_shards"][0]), p]), "full buffer")


@pytest.mark.parametrize("opt", ["sgd", "sgd-momentum"])
def test_stateless_and_one_state_optimizers_above_the_launch_cap(opt):
    """SGD without momentum keeps no state (exp_avg and exp_avg_sq are NULL) and
    its copies in the step's trip; with momentum it keeps one buffer and splits
    them out.  A shard above 2^26 elements is stepped in slices either way and
    matches the oracle on every element."""
    import numpy as np
    import oracle
    from parity import assert_bits_equal, oracle_chunks
    world, rank = 2, 0
    S = (1 << 26) + 77
    momentum = 0.9 if opt == "sgd-momentum" else 0.0
    hp = ss.OptimHP.sgd(lr=1e-2, momentum=momentum, weight_decay=1e-4, step=2)
    u = _units(world, rank, [S], torch.float16, torch.float16, 51)[0]
    if momentum == 0.0:
        u["exp_avg"] = u["exp_avg_sq"] = None
    else:
        u["exp_avg_sq"] = None
    gs = [np_of(g[:S]) for g in u["rank_grads"]]
    p = np_of(u["master"])
    buf = np_of(u["exp_avg"]) if momentum else None
    ss.fsdp_step_units([u], rank, True, hp)
    torch.cuda.synchronize()
    o = oracle.opt("sgd", step=2, lr=1e-2, momentum=momentum, weight_decay=1e-4)
    comp = np.empty(S, np.uint16)

    def step(lo, hi):
        g32 = oracle.grad_average(gs, lo, hi - lo, "f16", True)
        oracle.sgd(p[lo:hi], buf[lo:hi] if momentum else None, g32, o)
        comp[lo:hi] = oracle.cast(p[lo:hi], "f16")

    oracle_chunks(S, step)
    assert_bits_equal(np_of(u["master"]), p, "master")
    if momentum:
        assert_bits_equal(np_of(u["exp_avg"]), buf, "momentum buffer")
    assert_bits_equal(np_of(u["full"]), np.concatenate([comp, np_of(u["peer_shards"][1])]), "full buffer")
