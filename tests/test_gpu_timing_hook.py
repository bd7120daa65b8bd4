"""GPU: the profiling hook fsdp_time_next_launch.

The armed start/stop events ride on the next kernel the thread enqueues through
the library (its own dispatch packet), and are consumed by the next entry point
that returns.  Checked here: the step launch of a unit call is timed whether the
peers' copies run in its trip or in a launch of their own, and a host-only call
between arming and the launch consumes the pair (nothing is timed).
"""
import ctypes

import pytest
import torch

import sharded_state_amd as ss
from sharded_state_amd import _native as N

pytestmark = pytest.mark.gpu


class Events:
    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipGetLastError.restype = ctypes.c_int
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            self.ev.append(e)

    def elapsed(self, i, j):
        """(status, ms); a failed query's error is cleared so later HIP calls see none."""
        out = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[i], self.ev[j])
        if rc != 0:
            self.hip.hipGetLastError()
        return rc, out.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def _unit(world, S, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return dict(master=torch.randn(S, device="cuda", generator=g) * 0.02,
                exp_avg=torch.zeros(S, device="cuda"), exp_avg_sq=torch.zeros(S, device="cuda"),
                rank_grads=[(torch.randn(world * S, device="cuda", generator=g) * 1e-3).half() for _ in range(world)],
                peer_shards=[None] + [torch.randn(S, device="cuda", generator=g).half() for _ in range(world - 1)],
                full=torch.empty(world * S, dtype=torch.float16, device="cuda"))


@pytest.mark.parametrize("S", [1 << 20, 1 << 25])
def test_step_launch_is_timed(S):
    """1 Mi shard elements: the copies in the step's trip; 32 Mi: in a launch
    of their own.  Either way the armed events time the step launch."""
    world = 2
    split = ss.unit_gather_split(torch.float32, 2, S)
    assert split == (S >= 1 << 24)
    u = _unit(world, S, 3)
    call = ss.prepare_step_units([u], 0, True, ss.AdamWHP())
    call()                                          # warm
    torch.cuda.synchronize()
    ev = Events(2)
    lib = N.lib()
    assert lib.fsdp_time_next_launch(ev.ev[0], ev.ev[1]) == 0
    call()
    torch.cuda.synchronize()
    rc, ms = ev.elapsed(0, 1)
    ev.close()
    assert rc == 0
    # the step launch moves 30 B (split) or 34 B per shard element; well under a second, above 1 us
    assert 1e-3 < ms < 1000.0, ms


def test_host_call_consumes_the_armed_events():
    world, S = 2, 1 << 16
    u = _unit(world, S, 4)
    call = ss.prepare_step_units([u], 0, True, ss.AdamWHP())
    ev = Events(2)
    lib = N.lib()
    assert lib.fsdp_time_next_launch(ev.ev[0], ev.ev[1]) == 0
    ss.fsdp_layout([S * world], world)              # an entry point that returns: the pair is consumed
    call()                                          # not timed
    torch.cuda.synchronize()
    rc, _ = ev.elapsed(0, 1)
    ev.close()
    assert rc != 0                                   # never recorded
    torch.zeros(1, device="cuda").add_(1)            # the stream is healthy afterwards
    torch.cuda.synchronize()
