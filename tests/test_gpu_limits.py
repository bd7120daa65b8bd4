"""GPU parity at the limits of the interface.

* world = FSDP_MAX_WORLD (128) simulated ranks through the generic kernel, with
  the fused all-gather (127 peer copies) and through the separate reduce-scatter;
* a shard of more than 2**31 elements (64-bit element indexing end to end:
  tile numbers, vector and byte offsets), every element against the oracle;
* the grid-stride kernels past their one-trip grid (2048 workgroups per CU):
  a reduce-scatter of 2**30 + 12345 elements with fp32 output (group layout)
  and a gather of one 2**29 + 4099-element fp32 shard (over 2 GiB), where
  lanes take a second trip, every element compared.
"""
import numpy as np
import pytest
import torch

import oracle
import sharded_state_amd as ss
from parity import assert_bitexact, assert_bits_equal, np_of, oracle_chunks
from sharded_state_amd import _native as N

pytestmark = pytest.mark.gpu


def test_max_world_fused_step_and_gather():
    world = N.MAX_WORLD
    S = 263                                        # ragged: not a multiple of 8
    g = torch.Generator(device="cpu").manual_seed(3)
    grads = [(torch.randn(world * S, generator=g) * 1e-3).to(torch.float16).cuda() for _ in range(world)]
    master0 = (torch.randn(world * S, generator=g) * 0.02)
    peers = [(torch.randn(S, generator=g) * 0.02).to(torch.float16).cuda() for _ in range(world)]
    hp = ss.AdamWHP(step=3)
    gs = [np_of(x) for x in grads]
    h = oracle.hp(step=3)
    for rank in (0, 77, world - 1):
        sl = slice(rank * S, (rank + 1) * S)
        p = master0[sl].clone().cuda()
        m = torch.zeros(S, device="cuda")
        v = torch.zeros(S, device="cuda")
        full = torch.empty(world * S, dtype=torch.float16, device="cuda")
        ss.fsdp_step_unit(p, m, v, grads, rank, True, hp, [None if q == rank else peers[q] for q in range(world)],
                          full)
        rs = ss.fsdp_reduce_scatter_local(grads, rank, True, shard_numel=S)
        torch.cuda.synchronize()
        op, om, ov = np_of(master0[sl]), np.zeros(S, np.float32), np.zeros(S, np.float32)
        gshard, comp = oracle.rank_step(gs, rank, op, om, ov, h, "f16", True, "f16")
        assert_bitexact(np_of(rs), gshard, "reduce-scatter, rank %d of 128" % rank)
        assert_bitexact(np_of(p), op, "master, rank %d of 128" % rank)
        assert_bitexact(np_of(v), ov, "exp_avg_sq, rank %d of 128" % rank)
        f = np_of(full)
        assert_bitexact(f[sl], comp, "own slot, rank %d" % rank)
        want = np.concatenate([comp if q == rank else np_of(peers[q]) for q in range(world)])
        assert_bitexact(f, want, "gathered full buffer, rank %d" % rank)


def test_world_above_max_is_rejected():
    g = [torch.zeros(16, device="cuda") for _ in range(N.MAX_WORLD + 1)]
    with pytest.raises(ss.FsdpError):
        ss.fsdp_reduce_scatter_local(g, 0, True, shard_numel=0)


def test_shard_of_more_than_2_31_elements():
    """One rank (N = 1) with a shard of 2**31 + 4099 elements: fp16 gradient,
    fp32 master / m / v (8.6 GB each), bf16 compute copy written into the
    (single-slot) full buffer."""
    S = (1 << 31) + 4099                            # ragged tail past 2**31
    free, total = torch.cuda.mem_get_info()
    need = S * (2 + 12 + 2) + (1 << 30)
    if free < need:
        pytest.skip("needs %.1f GB of free device memory, %.1f GB free" % (need / 1e9, free / 1e9))
    print("S =", S, flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    grad = torch.empty(S, dtype=torch.float16, device="cuda")
    master = torch.empty(S, device="cuda")
    chunk = 1 << 28
    for lo in range(0, S, chunk):                   # fill in chunks (no fp32 temporary of 8.6 GB)
        hi = min(S, lo + chunk)
        grad[lo:hi] = (torch.randn(hi - lo, device="cuda", generator=g) * 1e-3).to(torch.float16)
        master[lo:hi] = torch.randn(hi - lo, device="cuda", generator=g) * 0.02
    m = torch.zeros(S, device="cuda")
    v = torch.zeros(S, device="cuda")
    g0, pm = np_of(grad), np_of(master)
    full = torch.empty(S, dtype=torch.bfloat16, device="cuda")
    ss.fsdp_step_units([dict(master=master, exp_avg=m, exp_avg_sq=v, rank_grads=[grad], full=full,
                             peer_shards=[None])], 0, True, ss.AdamWHP(step=1))
    torch.cuda.synchronize()
    print("step done; oracle on every element", flush=True)
    h = oracle.hp(step=1)
    mm, vm = np.zeros(S, np.float32), np.zeros(S, np.float32)
    comp = np.empty(S, np.uint16)

    def step(lo, hi):
        oracle.adamw(pm[lo:hi], mm[lo:hi], vm[lo:hi], oracle.to_f32(g0[lo:hi], "f16"), h)
        comp[lo:hi] = oracle.cast(pm[lo:hi], "bf16")

    oracle_chunks(S, step)
    del g0
    assert_bits_equal(np_of(master), pm, "master")
    assert_bits_equal(np_of(m), mm, "exp_avg")
    assert_bits_equal(np_of(v), vm, "exp_avg_sq")
    assert_bits_equal(np_of(full), comp, "compute copy in the full buffer")


def _need(nbytes):
    free, _ = torch.cuda.mem_get_info()
    if free < nbytes + (1 << 30):
        pytest.skip("needs %.1f GB of free device memory, %.1f GB free" % (nbytes / 1e9, free / 1e9))


def test_reduce_scatter_beyond_one_trip_of_its_grid():
    """N = 1, fp16 gradient reduced to fp32: 2**30 + 12345 elements are more
    vectors than the capped grid has lanes (256 CUs x 2048 x 256 = 2**27), so
    the last groups are reduced on a second trip of the grid-stride loop."""
    S = (1 << 30) + 12345
    _need(S * (2 + 4))
    print("S =", S, flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(13)
    grad = torch.empty(S, dtype=torch.float16, device="cuda")
    chunk = 1 << 28
    for lo in range(0, S, chunk):
        hi = min(S, lo + chunk)
        grad[lo:hi] = (torch.randn(hi - lo, device="cuda", generator=g) * 1e-3).to(torch.float16)
    out = ss.fsdp_reduce_scatter_local([grad], 0, True)
    torch.cuda.synchronize()
    g0 = np_of(grad)
    ref = np.empty(S, np.float32)

    def rs(lo, hi):
        ref[lo:hi] = oracle.reduce_scatter([g0[lo:hi]], 0, "f16", True)

    oracle_chunks(S, rs)
    assert_bits_equal(np_of(out), ref, "reduce-scatter, two trips")


def test_gather_beyond_one_trip_of_its_grid():
    """One fp32 shard of 2**29 + 4099 elements (2.1 GB) gathered into a
    one-slot full buffer: more 16-byte vectors than the grid's lanes, so the
    copy takes a second trip; the result is the shard, byte for byte."""
    S = (1 << 29) + 4099
    _need(S * 8)
    print("S =", S, flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(17)
    shard = torch.empty(S, device="cuda")
    chunk = 1 << 28
    for lo in range(0, S, chunk):
        hi = min(S, lo + chunk)
        shard[lo:hi] = torch.randn(hi - lo, device="cuda", generator=g)
    full = ss.fsdp_unshard_gather([shard])
    torch.cuda.synchronize()
    sh = np_of(shard)
    assert_bits_equal(np_of(full), oracle.gather([sh], "f32"), "gather, two trips")
