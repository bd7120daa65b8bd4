"""fsdp_offload_step_units_noalloc, the offloaded step without a device
gradient shard (its chunks go through the library's per-device scratch), called
through the C ABI and compared bit for bit with fsdp_offload_step_units on the
same inputs: three calls in a row on one device, each smaller than the one
before (so every call after the first finds the scratch holding the previous
call's bytes), one with more chunks than the scratch has events.  Also: a
chunk larger than the scratch and a non-NULL grad_shard_dev are refused before
anything is enqueued.
"""
import ctypes

import pytest
import torch

import sharded_state_amd as ss
from parity import assert_bits_equal, np_of
from sharded_state_amd import _native as N

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _state(S, seed, avg_dt, cdt, device_grad):
    g = torch.Generator().manual_seed(seed)
    pin = dict(pin_memory=True)
    st = dict(master=(torch.randn(S, generator=g) * 0.02).pin_memory(),
              exp_avg=(torch.randn(S, generator=g) * 1e-4).abs().pin_memory(),
              exp_avg_sq=(torch.randn(S, generator=g) * 1e-4).abs().pin_memory(),
              grad_host=torch.empty(S, dtype=avg_dt, **pin), compute_host=torch.empty(S, dtype=cdt, **pin),
              compute_dev=torch.empty(S, dtype=cdt, device="cuda"),
              grad_dev=torch.empty(S, dtype=avg_dt, device="cuda") if device_grad else None)
    return st


def _table(states, gptrs):
    t = (N.OffloadUnit * len(states))()
    for k, (st, gp) in enumerate(zip(states, gptrs)):
        t[k] = N.OffloadUnit(st["master"].data_ptr(), st["exp_avg"].data_ptr(), st["exp_avg_sq"].data_ptr(), gp,
                             st["grad_dev"].data_ptr() if st["grad_dev"] is not None else None,
                             st["grad_host"].data_ptr(), st["compute_host"].data_ptr(), st["compute_dev"].data_ptr(),
                             st["master"].numel())
    return t


# (world, rank, grad dtype, fp32 reduce, compute dtype, shard sizes, chunk_numel, threads, copy stream)
CALLS = [
    (2, 1, "f32", True, "f16", [5_000_011, 3_000_017], 0, 8, False),      # 4 Mi-element chunks (16 MiB)
    (2, 0, "f16", True, "bf16", [3_000_017, 1_000_003], 8192, 4, True),   # 490 chunks: events reused
    (8, 5, "bf16", False, "bf16", [12_345], 1000, 2, True),               # 16-bit average, N = 8
]


def test_noalloc_offload_matches_the_allocating_entry_point():
    L = N.lib()
    hp = N.AdamWHP(step=2)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for call, (world, rank, gdt, fp32r, cdt, sizes, chunk, threads, use_cs) in enumerate(CALLS):
        print("case no-alloc offload call %d: N=%d rank %d %s sizes %s chunk %d" % (call, world, rank, gdt, sizes,
                                                                                   chunk), flush=True)
        avg_dt = torch.float32 if (fp32r or gdt == "f32") else DT[gdt]
        gen = torch.Generator(device="cuda")
        gen.manual_seed(call)
        grads = [[(torch.randn(world * S, device="cuda", generator=gen) * 1e-3).to(DT[gdt]) for _ in range(world)]
                 for S in sizes]
        gptrs = [N.ptr_array([g.data_ptr() for g in gs]) for gs in grads]
        ref = [_state(S, 10 * call + k, avg_dt, DT[cdt], True) for k, S in enumerate(sizes)]
        got = [_state(S, 10 * call + k, avg_dt, DT[cdt], False) for k, S in enumerate(sizes)]
        cs = torch.cuda.Stream() if use_cs else None
        cst = ctypes.c_void_p(cs.cuda_stream) if cs is not None else None
        args = (len(sizes), world, rank, ss.dtype_code(DT[gdt]), int(fp32r), ss.dtype_code(DT[cdt]), chunk,
                ctypes.byref(hp), threads, stream, cst)
        N.check("fsdp_offload_step_units", L.fsdp_offload_step_units(_table(ref, gptrs), *args))
        N.check("fsdp_offload_step_units_noalloc", L.fsdp_offload_step_units_noalloc(_table(got, gptrs), *args))
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(ref, got)):
            for key in ("master", "exp_avg", "exp_avg_sq", "grad_host", "compute_host", "compute_dev"):
                assert_bits_equal(np_of(b[key]), np_of(a[key]), "call %d unit %d %s" % (call, k, key))


def test_noalloc_offload_refuses_oversized_chunks_and_a_device_gradient_shard():
    L = N.lib()
    hp = N.AdamWHP()
    S = 4096
    gs = [torch.zeros(2 * S, dtype=torch.float16, device="cuda") for _ in range(2)]
    gp = N.ptr_array([g.data_ptr() for g in gs])
    st = _state(S, 0, torch.float32, torch.float16, True)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    too_big = N.OFFLOAD_SCRATCH_BYTES // 4 + 8            # fp32 average: one 8-element group past the scratch
    no_dev = dict(st, grad_dev=None)
    rc = L.fsdp_offload_step_units_noalloc(_table([no_dev], [gp]), 1, 2, 0, N.F16, 1, N.F16, too_big,
                                           ctypes.byref(hp), 2, stream, None)
    assert rc == N.E_SIZE and "scratch" in L.fsdp_last_error().decode()
    rc = L.fsdp_offload_step_units_noalloc(_table([st], [gp]), 1, 2, 0, N.F16, 1, N.F16, 0, ctypes.byref(hp), 2,
                                           stream, None)
    assert rc == N.E_INVAL and "grad_shard_dev must be NULL" in L.fsdp_last_error().decode()
    torch.cuda.synchronize()


def test_noalloc_offload_calls_from_two_threads_take_the_scratch_in_turn():
    """Two host threads call the no-allocation step on one device at once, on
    two streams, with different units: the library's per-device lock serializes
    them, so each gets the same bytes as the allocating entry point."""
    import threading
    L = N.lib()
    hp = N.AdamWHP(step=3)
    world, rank, gdt, fp32r, cdt = 2, 1, "bf16", False, "bf16"
    avg_dt = DT[gdt]
    jobs = []
    for t in range(2):
        S = 2_000_003 + 5 * t
        gen = torch.Generator(device="cuda")
        gen.manual_seed(50 + t)
        grads = [(torch.randn(world * S, device="cuda", generator=gen) * 1e-3).to(DT[gdt]) for _ in range(world)]
        gp = N.ptr_array([g.data_ptr() for g in grads])
        ref = _state(S, 60 + t, avg_dt, DT[cdt], True)
        got = _state(S, 60 + t, avg_dt, DT[cdt], False)
        jobs.append(dict(S=S, grads=grads, gp=gp, ref=ref, got=got, stream=torch.cuda.Stream()))
    stream0 = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for j in jobs:
        N.check("fsdp_offload_step_units", L.fsdp_offload_step_units(
            _table([j["ref"]], [j["gp"]]), 1, world, rank, ss.dtype_code(DT[gdt]), int(fp32r), ss.dtype_code(DT[cdt]),
            65536, ctypes.byref(hp), 4, stream0, None))
    torch.cuda.synchronize()
    rcs = [None, None]

    def run(k):
        j = jobs[k]
        with torch.cuda.device(0):
            rcs[k] = L.fsdp_offload_step_units_noalloc(
                _table([j["got"]], [j["gp"]]), 1, world, rank, ss.dtype_code(DT[gdt]), int(fp32r),
                ss.dtype_code(DT[cdt]), 65536, ctypes.byref(hp), 4, ctypes.c_void_p(j["stream"].cuda_stream), None)

    threads = [threading.Thread(target=run, args=(k,)) for k in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert rcs == [N.OK, N.OK], rcs
    for k, j in enumerate(jobs):
        for key in ("master", "exp_avg", "exp_avg_sq", "grad_host", "compute_host", "compute_dev"):
            assert_bits_equal(np_of(j["got"][key]), np_of(j["ref"][key]), "thread %d %s" % (k, key))
