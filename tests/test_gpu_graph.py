"""GPU: the unit step captured in a HIP graph.

Launch-bound callers (many small units, tight loops) can capture a step once
and replay it.  The library enqueues kernels only (no memset or allocation, no
host synchronisation), so a captured step must replay exactly like the eager
call.  Each replay here is followed by eager work of the program's own, a
synchronisation, and the eager call on a copy of the inputs; every replay's
outputs are compared bit for bit with that copy's.  Both forms of the gather
are captured: the copies in the step's trip (small units) and the copies in a
launch of their own (2^24+ shard elements).
"""
import pytest
import torch

import sharded_state_amd as ss

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _units(world, rank, sizes, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = []
    for S in sizes:
        out.append(dict(
            master=torch.randn(S, device="cuda", generator=g) * 0.02,
            exp_avg=torch.randn(S, device="cuda", generator=g) * 1e-3,
            exp_avg_sq=torch.rand(S, device="cuda", generator=g) * 1e-6,
            rank_grads=[(torch.randn(world * S, device="cuda", generator=g) * 1e-3).half() for _ in range(world)],
            peer_shards=[None if q == rank else torch.randn(S, device="cuda", generator=g).half()
                         for q in range(world)],
            full=torch.zeros(world * S, dtype=torch.float16, device="cuda")))
    return out


def _clone(units):
    return [dict(u, master=u["master"].clone(), exp_avg=u["exp_avg"].clone(), exp_avg_sq=u["exp_avg_sq"].clone(),
                 full=u["full"].clone()) for u in units]


@pytest.mark.parametrize("sizes", [[4099, 70_000, 1 << 18], [(1 << 23) + 8, (1 << 23) + 64]])
def test_captured_step_replays_like_the_eager_step(sizes):
    world, rank = 2, 1
    hp = ss.AdamWHP(1e-3, 0.9, 0.999, 1e-8, 0.01, 5)
    print("case", sizes, "split", ss.unit_gather_split(torch.float32, 2, sum(sizes)), flush=True)
    a = _units(world, rank, sizes, 9)
    b = _clone(a)
    eager = ss.prepare_step_units(b, rank, True, hp)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                    # warm up on a side stream, as capture wants
        w = _clone(a)
        ss.fsdp_step_units(w, rank, True, hp)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del w
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = ss.prepare_step_units(a, rank, True, hp)   # binds the capture stream
        captured()
    torch.cuda.synchronize()
    scratch = torch.ones(1 << 20, device="cuda")
    for replay in range(3):
        graph.replay()
        scratch.mul_(1.5).add_(replay)               # the program's own eager work between replays
        torch.cuda.synchronize()
        eager()
        torch.cuda.synchronize()
        for k, (ua, ub) in enumerate(zip(a, b)):
            for key in ("master", "exp_avg", "exp_avg_sq", "full"):
                assert torch.equal(_bits(ua[key]), _bits(ub[key])), (replay, k, key)
