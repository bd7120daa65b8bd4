"""Guard bands around every output of every entry point that writes device
memory: a known byte pattern before and after each output buffer must be
intact after the call, and the outputs must still match the oracle.  The
cases reach every indexing regime of the kernels: a unit above the 2^26-element
launch cap (stepped in slices whose pointers start further in), a launch of
at least 2^24 shard elements (the peers' copies in a launch of their own),
several units packed into one launch, ragged shard sizes (the single-element
tail after the last whole 512-element group), buffers off the 16-byte grid
(the whole unit on the per-element path), N = 3 (the generic kernel), N = 8
with the persistent own copy, 16-bit state and SGD without state.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import sharded_state_amd as ss
from guards import Guarded
from parity import assert_bits_equal, assert_compute_close, dt_name, np_of, oracle_rank_step_threaded
from sharded_state_amd import _native as N

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _gen(seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


def _randn(n, dtype, scale, seed):
    return (torch.randn(n, device="cuda", generator=_gen(seed)) * scale).to(dtype)


def _off(off, dtype):
    """The case's byte offset where the element size divides it, else 0 (a
    2-byte offset misaligns the 16-bit outputs and leaves fp32 state aligned)."""
    return off if off % torch.empty(0, dtype=dtype).element_size() == 0 else 0


# (name, world, rank, [shard sizes], grad dtype, fp32 reduce, compute dtype, state dtype, optimizer,
#  persistent copy, byte offset of the outputs)
STEP_CASES = [
    ("fused-two-units", 2, 1, [12345, 4099], "f16", True, "f16", "f32", "adamw", False, 0),
    ("split-copies", 2, 0, [(1 << 24) + 1003], "f16", True, "f16", "f32", "adamw", False, 0),
    ("sliced-above-cap", 2, 1, [(1 << 26) + 1003], "bf16", False, "bf16", "f32", "adamw", False, 0),
    ("packed-six", 2, 0, [1_000_003 + 8 * k for k in range(6)], "f16", True, "f16", "f32", "adamw", False, 0),
    ("n8-persistent", 8, 7, [(1 << 20) + 517], "f16", True, "f16", "f32", "adamw", True, 0),
    ("generic-n3", 3, 2, [4099 + 7, 333], "bf16", False, "bf16", "f32", "adamw", False, 0),
    ("unaligned", 2, 0, [12345], "f16", True, "f16", "f32", "adamw", False, 4),
    ("unaligned-16bit-out", 2, 1, [20011], "bf16", False, "bf16", "f32", "adamw", True, 2),
    ("state-bf16", 2, 1, [100_003, 4096], "bf16", False, "bf16", "bf16", "adamw", False, 0),
    ("state-bf16-n8", 8, 3, [65_541], "bf16", False, "bf16", "bf16", "adamw", False, 0),
    ("sgd-no-state", 2, 0, [(1 << 24) + 77], "f16", True, "f16", "f32", "sgd", False, 0),
    ("sgd-momentum", 4, 2, [50_021], "f16", True, "f16", "f32", "sgd-momentum", False, 0),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_step_units_writes_nothing_outside_its_outputs(case):
    name, world, rank, sizes, gdt, fp32r, cdt, sdt, opt, persistent, off = case
    print("case guard step", name, flush=True)
    state16 = sdt != "f32"
    hp = ss.AdamWHP(step=3)
    ohp = None
    if opt == "sgd":
        ohp = ss.OptimHP.sgd(lr=1e-2, weight_decay=1e-4, step=3)
    elif opt == "sgd-momentum":
        ohp = ss.OptimHP.sgd(lr=1e-2, momentum=0.9, weight_decay=1e-4, step=3)
    n_states = ohp.n_states if ohp is not None else 2
    units, guards, refs = [], [], []
    for k, S in enumerate(sizes):
        seed = 1000 * k
        grads = [_randn(world * S, DT[gdt], 1e-3, seed + q) for q in range(world)]
        st_dt = DT[sdt]
        p0 = _randn(S, st_dt, 0.02, seed + 100)
        m0 = _randn(S, st_dt, 1e-4, seed + 101).abs() if n_states >= 1 else None
        v0 = _randn(S, st_dt, 1e-4, seed + 102).abs() if n_states >= 2 else None
        so, co = _off(off, st_dt), _off(off, DT[cdt])
        gp = Guarded(S, st_dt, so, init=p0)
        gm = Guarded(S, st_dt, so, init=m0) if m0 is not None else None
        gv = Guarded(S, st_dt, so, init=v0) if v0 is not None else None
        gfull = Guarded(world * S, DT[cdt], co)
        gpers = Guarded(S, DT[cdt], co) if persistent else None
        peers = [None if q == rank else _randn(S, DT[cdt], 0.02, seed + 200 + q) for q in range(world)]
        u = dict(master=gp.t, rank_grads=grads, peer_shards=peers, full=gfull.t)
        if gm is not None:
            u["exp_avg"] = gm.t
        if gv is not None:
            u["exp_avg_sq"] = gv.t
        if gpers is not None:
            u["compute_shard"] = gpers.t
        units.append(u)
        guards.append([x for x in (gp, gm, gv, gfull, gpers) if x is not None])
        sl = slice(rank * S, (rank + 1) * S)
        refs.append(dict(grads=[np_of(g[sl]) for g in grads], p=np_of(p0),
                         m=np_of(m0) if m0 is not None else None, v=np_of(v0) if v0 is not None else None,
                         peers=[None if x is None else np_of(x) for x in peers]))
    ss.fsdp_step_units(units, rank, fp32r, hp if ohp is None else ohp)
    torch.cuda.synchronize()
    for k, (S, u, gl, r) in enumerate(zip(sizes, units, guards, refs)):
        for g in gl:
            g.check("%s unit %d" % (name, k))
        if opt == "adamw" and not state16:
            avg, comp = oracle_rank_step_threaded(r["grads"], r["p"], r["m"], r["v"], oracle.hp(step=3), gdt, fp32r,
                                                  cdt)
        else:
            avg = oracle.grad_average(r["grads"], 0, S, gdt, fp32r)
            g32 = avg if avg.dtype == np.float32 else oracle.to_f32(avg, gdt)
            if state16:
                oracle.adamw16(r["p"], r["m"], r["v"], g32, oracle.hp(step=3), sdt)
                comp = r["p"]
            else:
                o = oracle.opt("sgd", step=3, lr=1e-2, weight_decay=1e-4,
                               momentum=0.9 if opt == "sgd-momentum" else 0.0)
                oracle.sgd(r["p"], r["m"], g32, o)
                comp = oracle.cast(r["p"], cdt)
        assert_bits_equal(np_of(u["master"]), r["p"], "%s master %d" % (name, k))
        if n_states >= 1:
            assert_bits_equal(np_of(u["exp_avg"]), r["m"], "%s exp_avg %d" % (name, k))
        if n_states >= 2:
            assert_bits_equal(np_of(u["exp_avg_sq"]), r["v"], "%s exp_avg_sq %d" % (name, k))
        ref_full = oracle.gather([comp if q == rank else r["peers"][q] for q in range(world)], cdt)
        assert_compute_close(np_of(u["full"]), ref_full, cdt, "%s full %d" % (name, k))
        if persistent:
            assert_compute_close(np_of(u["compute_shard"]), comp, cdt, "%s persistent %d" % (name, k))


@pytest.mark.parametrize("world,S,gdt,fp32r,off", [(2, 12345, "f16", True, 0), (3, 4099, "bf16", False, 2),
                                                    (8, 65_543, "f16", True, 4), (2, (1 << 20) + 3, "f32", True, 0)])
def test_reduce_scatter_writes_nothing_outside_its_output(world, S, gdt, fp32r, off):
    print("case guard reduce-scatter", world, S, gdt, flush=True)
    rank = world - 1
    grads = [_randn(world * S, DT[gdt], 1e-3, 7 + q) for q in range(world)]
    odt = "f32" if (fp32r or gdt == "f32") else gdt
    out = Guarded(S, DT[odt], _off(off, DT[odt]))
    ss.fsdp_reduce_scatter_local(grads, rank, fp32r, out=out.t, shard_numel=S)
    out.check("reduce-scatter")
    ref = oracle.reduce_scatter([np_of(g) for g in grads], rank, gdt, fp32r)
    assert_bits_equal(np_of(out.t), ref, "reduce-scatter")


@pytest.mark.parametrize("off", [0, 4])
def test_sharded_adamw_writes_nothing_outside_its_outputs(off):
    print("case guard sharded_adamw", off, flush=True)
    world, rank, S = 2, 1, 40_009
    grads = [_randn(world * S, torch.float16, 1e-3, 30 + q) for q in range(world)]
    p0 = _randn(S, torch.float32, 0.02, 40)
    gp, gm, gv = Guarded(S, torch.float32, off, init=p0), Guarded(S, torch.float32, off), Guarded(S, torch.float32, off)
    gm.t.zero_()
    gv.t.zero_()
    gc = Guarded(S, torch.float16, off // 2)
    ss.fsdp_sharded_adamw(gp.t, gm.t, gv.t, grads, rank, True, ss.AdamWHP(), compute_shard=gc.t)
    for g, w in ((gp, "master"), (gm, "exp_avg"), (gv, "exp_avg_sq"), (gc, "compute")):
        g.check(w)
    sl = slice(rank * S, (rank + 1) * S)
    p, m, v = np_of(p0), np.zeros(S, np.float32), np.zeros(S, np.float32)
    _, comp = oracle_rank_step_threaded([np_of(g[sl]) for g in grads], p, m, v, oracle.hp(), "f16", True, "f16")
    assert_bits_equal(np_of(gp.t), p, "master")
    assert_bits_equal(np_of(gc.t), comp, "compute")


def test_gather_and_flatten_and_unflatten_write_nothing_outside_their_outputs():
    print("case guard gather / flatten / unflatten", flush=True)
    world, S = 3, 4099
    shards = [_randn(S, torch.float16, 1.0, 50 + q) for q in range(world)]
    full = Guarded(world * S, torch.float16, 2)
    ss.fsdp_unshard_gather(shards, full=full.t)
    full.check("gather")
    assert_bits_equal(np_of(full.t), oracle.gather([np_of(s) for s in shards], "f16"), "gather")

    shapes = [(1000, 999), (999,), (1,), (7, 3)]
    for dt, off in ((torch.float32, 0), (torch.float32, 4), (torch.bfloat16, 2)):
        tensors = [_randn(int(np.prod(s)), dt, 1.0, 60 + k).reshape(s) for k, s in enumerate(shapes)]
        numels = [t.numel() for t in tensors]
        P, Pp, _ = ss.fsdp_layout(numels, world)
        flat = Guarded(Pp, dt, off)
        ss.fsdp_flatten_pad(tensors, world, flat=flat.t)
        flat.check("flatten")
        name = dt_name(dt)
        assert_bits_equal(np_of(flat.t), oracle.flatten_pad([np_of(t).reshape(-1) for t in tensors], world, name),
                          "flatten")
        dsts = [Guarded(n, dt, off) for n in numels]
        views = (N.View * len(numels))()
        N.check("fsdp_unflatten_views", N.lib().fsdp_unflatten_views(
            N.i64_array(numels), len(numels), Pp, views, ctypes.c_void_p(flat.t.data_ptr()), ss.dtype_code(dt),
            N.ptr_array([d.t.data_ptr() for d in dsts]), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
        for k, (d, ref) in enumerate(zip(dsts, oracle.unflatten(np_of(flat.t), shapes, name))):
            d.check("unflatten %d" % k)
            assert_bits_equal(np_of(d.t), ref.reshape(-1), "unflatten %d" % k)


def test_offload_step_writes_nothing_outside_its_outputs():
    print("case guard offload", flush=True)
    world, rank, S = 2, 1, 100_003
    grads = [_randn(world * S, torch.bfloat16, 1e-3, 70 + q) for q in range(world)]
    p0 = _randn(S, torch.float32, 0.02, 80).cpu()
    hp_ = dict(device="cpu")
    hm, hv = Guarded(S, torch.float32, 4, **hp_), Guarded(S, torch.float32, 4, **hp_)
    hmaster = Guarded(S, torch.float32, 4, init=p0, **hp_)
    hm.t.zero_()
    hv.t.zero_()
    hgrad = Guarded(S, torch.bfloat16, 2, **hp_)
    hcomp = Guarded(S, torch.bfloat16, 2, **hp_)
    dgrad = Guarded(S, torch.bfloat16, 2)
    dcomp = Guarded(S, torch.bfloat16, 2)
    ss.fsdp_offload_step(hmaster.t, hm.t, hv.t, grads, rank, False, ss.AdamWHP(), dgrad.t, hgrad.t, hcomp.t, dcomp.t,
                         chunk_numel=4104, n_threads=3)
    torch.cuda.synchronize()
    for g, w in ((hmaster, "host master"), (hm, "host exp_avg"), (hv, "host exp_avg_sq"), (hgrad, "host grad"),
                 (hcomp, "host compute"), (dgrad, "device grad shard"), (dcomp, "device compute")):
        g.check(w)
    sl = slice(rank * S, (rank + 1) * S)
    p, m, v = np_of(p0), np.zeros(S, np.float32), np.zeros(S, np.float32)
    _, comp = oracle_rank_step_threaded([np_of(g[sl]) for g in grads], p, m, v, oracle.hp(), "bf16", False, "bf16")
    assert_bits_equal(np_of(hmaster.t), p, "offload master")
    assert_bits_equal(np_of(dcomp.t), comp, "offload compute")


def test_load_shard_writes_nothing_outside_its_destinations(tmp_path):
    print("case guard load_shard", flush=True)
    S, world, rank = 70_001, 2, 1
    numels = [2 * S - 1]                       # padded to 2S: shard S
    state = [_randn(S, torch.float32, 0.02, 90 + k) for k in range(3)]
    path = ss.shard_path(str(tmp_path / "unit"), rank)
    ss.save_shard(path, numels, world, rank, *state, step=4, hp=ss.AdamWHP(), compute_dtype=torch.bfloat16)
    dst = [Guarded(S, torch.float32, off) for off in (0, 4, 12)]
    ss.load_shard(path, *[d.t for d in dst])
    torch.cuda.synchronize()
    for k, (d, s) in enumerate(zip(dst, state)):
        d.check("load_shard %d" % k)
        assert_bits_equal(np_of(d.t), np_of(s), "load_shard %d" % k)
