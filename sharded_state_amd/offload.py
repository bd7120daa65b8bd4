"""CPU offload of the optimizer step: the fp32 master shard and the AdamW
moments live in host memory and the update runs on the host
("Fully Sharded Data Parallel: faster AI training with fewer GPUs",
"Adoption paths for FSDP", the fairseq --cpu-offload flag; "FSDP (Fully
Sharded Data Parallel)", "CPU Offloading").

Binding of fsdp_host_adamw and fsdp_offload_step (argument marshalling only:
the reduce-scatter runs in the library's HIP kernel, the update in its
multi-threaded host kernel, the copies on the caller's stream).
"""
import ctypes
import os

import torch

from . import _native as N
from ._native import AdamWHP, check
from .api import _dev, _grads, _own_hp, _reissue, _same_device, _stream, dtype_code

# Worker threads of the host update: the host's cores, at most 16.
DEFAULT_THREADS = max(1, min(16, os.cpu_count() or 1))


def _host(t, name, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.device.type != "cpu":
        raise ValueError("%s must be a host tensor, got %s" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t


def _vp(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else None)


def fsdp_host_adamw(master, exp_avg, exp_avg_sq, grad, hp, compute=None, n_threads=None):
    """AdamW on host tensors (master, exp_avg, exp_avg_sq fp32, updated in place;
    grad fp32/fp16/bf16; compute, if given, receives the rounded master)."""
    n = master.numel()
    for name, t in (("master", master), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        _host(t, name, torch.float32)
        if t.numel() != n:
            raise ValueError("%s has %d elements, master %d" % (name, t.numel(), n))
    _host(grad, "grad")
    if grad.numel() != n:
        raise ValueError("grad has %d elements, need %d" % (grad.numel(), n))
    cdt = N.F32
    if compute is not None:
        _host(compute, "compute")
        if compute.numel() != n:
            raise ValueError("compute has %d elements, need %d" % (compute.numel(), n))
        cdt = dtype_code(compute.dtype)
    if not isinstance(hp, AdamWHP):
        hp = AdamWHP(**hp)
    check("fsdp_host_adamw", N.lib().fsdp_host_adamw(
        _vp(master), _vp(exp_avg), _vp(exp_avg_sq), _vp(grad), dtype_code(grad.dtype), _vp(compute), cdt, n,
        ctypes.byref(hp), int(n_threads or DEFAULT_THREADS)))
    return compute


def _unit(master, exp_avg, exp_avg_sq, rank_grads, grad_shard_dev, grad_shard_host, compute_host, compute_dev,
          fp32_reduce, device_grad=True):
    """Check one unit's tensors; returns (OffloadUnit, grad dtype, compute dtype, keep-alive).
    Without device_grad (the no-allocation call) grad_shard_dev must be None."""
    S = master.numel()
    for name, t in (("master", master), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        _host(t, name, torch.float32)
        if t.numel() != S:
            raise ValueError("%s has %d elements, master %d" % (name, t.numel(), S))
    rank_grads, world, gdt = _grads(rank_grads, S)
    odt = torch.float32 if (fp32_reduce or gdt == torch.float32) else gdt
    if device_grad:
        _dev(grad_shard_dev, "grad_shard_dev")
        if grad_shard_dev.dtype != odt:
            raise TypeError("grad_shard_dev must be %s, got %s" % (odt, grad_shard_dev.dtype))
    elif grad_shard_dev is not None:
        raise ValueError("the no-allocation call takes no grad_shard_dev (its chunks live in the library's scratch)")
    _dev(compute_dev, "compute_dev")
    _host(grad_shard_host, "grad_shard_host", odt)
    _host(compute_host, "compute_host", compute_dev.dtype)
    for name, t in (("grad_shard_dev", grad_shard_dev), ("grad_shard_host", grad_shard_host),
                    ("compute_host", compute_host), ("compute_dev", compute_dev)):
        if t is not None and t.numel() != S:
            raise ValueError("%s has %d elements, need %d" % (name, t.numel(), S))
    _same_device(rank_grads + [compute_dev] + ([grad_shard_dev] if device_grad else []))
    gptr = N.ptr_array([g.data_ptr() for g in rank_grads])
    u = N.OffloadUnit(master.data_ptr(), exp_avg.data_ptr(), exp_avg_sq.data_ptr(), gptr,
                      grad_shard_dev.data_ptr() if device_grad else None, grad_shard_host.data_ptr(),
                      compute_host.data_ptr(), compute_dev.data_ptr(), S)
    return u, world, gdt, compute_dev.dtype, gptr


def _hp(hp):
    return hp if isinstance(hp, AdamWHP) else AdamWHP(**hp)


def _cstream(copy_stream):
    return ctypes.c_void_p(copy_stream.cuda_stream) if copy_stream is not None else None


def fsdp_offload_step(master, exp_avg, exp_avg_sq, rank_grads, rank, fp32_reduce, hp, grad_shard_dev,
                      grad_shard_host, compute_host, compute_dev, chunk_numel=0, n_threads=None, stream=None,
                      copy_stream=None):
    """One offloaded rank step: device reduce-scatter of block `rank`, chunked
    copy to the host, host AdamW on the host master/m/v, copy of the compute
    shard to compute_dev (on copy_stream when given).  Returns once the host
    update is done; the copies to the device are enqueued."""
    u, world, gdt, cdt, keep = _unit(master, exp_avg, exp_avg_sq, rank_grads, grad_shard_dev, grad_shard_host,
                                     compute_host, compute_dev, fp32_reduce)
    hp = _hp(hp)
    device = compute_dev.device
    with torch.cuda.device(device):
        check("fsdp_offload_step", N.lib().fsdp_offload_step(
            u.master, u.exp_avg, u.exp_avg_sq, u.rank_grads, world, int(rank), dtype_code(gdt),
            int(bool(fp32_reduce)), u.grad_shard_dev, u.grad_shard_host, u.compute_host, u.compute_dev,
            dtype_code(cdt), u.shard_numel, int(chunk_numel), ctypes.byref(hp), int(n_threads or DEFAULT_THREADS),
            _stream(stream, device), _cstream(copy_stream)))
    del keep
    return compute_dev


def prepare_offload_step_units(units, rank, fp32_reduce, hp, chunk_numel=0, n_threads=None, stream=None,
                               copy_stream=None):
    """Marshal a batch once; returns a callable that runs
    fsdp_offload_step_units on it: call(step=t) takes step t, call(stream=s)
    runs on stream s (default: the stream given here, else the current
    stream at the time of the call); call.hp holds the hyper-parameters it
    reads.  units: (OffloadState, rank_grads, compute_dev) triples, each state
    at most once."""
    if not units:
        raise ValueError("units is empty")
    table = (N.OffloadUnit * len(units))()
    keep = []
    meta = None
    for k, (st, grads, cdev) in enumerate(units):
        u, world, gdt, cdt, gptr = _unit(st.master, st.exp_avg, st.exp_avg_sq, grads, st.grad_dev, st.grad_host,
                                         st.compute_host, cdev, st.fp32_reduce)
        if meta is None:
            meta = (world, gdt, cdt, st.fp32_reduce, cdev.device)
        elif meta != (world, gdt, cdt, st.fp32_reduce, cdev.device):
            raise ValueError("unit %d: world, dtypes, fp32_reduce and device must match unit 0" % k)
        table[k] = u
        keep.append((gptr, st, list(grads), cdev))    # the C side reads these at every call
    world, gdt, cdt, fp32, device = meta
    hp = _own_hp(_hp(hp))
    L = N.lib()
    cst = _cstream(copy_stream)
    args = (table, len(units), world, int(rank), dtype_code(gdt), int(bool(fp32)), dtype_code(cdt),
            int(chunk_numel), ctypes.byref(hp), int(n_threads or DEFAULT_THREADS), None, cst)

    def fn(*a):   # a ends with the stream; the copy stream follows it
        return L.fsdp_offload_step_units(*a, cst)

    call = _reissue(fn, "fsdp_offload_step_units", args[:-1], hp, stream, device)
    call.keep = (keep, table, hp, copy_stream)
    return call


def fsdp_offload_step_units_noalloc(units, rank, fp32_reduce, hp, chunk_numel=0, n_threads=None, stream=None,
                                    copy_stream=None):
    """fsdp_offload_step_units without a device gradient shard: each chunk is
    reduce-scattered into the library's fixed per-device scratch
    (OFFLOAD_SCRATCH_BYTES) and copied to the host from there; no device
    memory is allocated.  units: (OffloadState made with device_grad=False,
    rank_grads, compute_dev) triples.  Calls that overlap on one device race."""
    if not units:
        raise ValueError("units is empty")
    table = (N.OffloadUnit * len(units))()
    keep, meta = [], None
    for k, (st, grads, cdev) in enumerate(units):
        u, world, gdt, cdt, gptr = _unit(st.master, st.exp_avg, st.exp_avg_sq, grads, st.grad_dev, st.grad_host,
                                         st.compute_host, cdev, st.fp32_reduce, device_grad=False)
        if meta is None:
            meta = (world, gdt, cdt, st.fp32_reduce, cdev.device)
        elif meta != (world, gdt, cdt, st.fp32_reduce, cdev.device):
            raise ValueError("unit %d: world, dtypes, fp32_reduce and device must match unit 0" % k)
        table[k] = u
        keep.append(gptr)
    world, gdt, cdt, fp32, device = meta
    hp = _hp(hp)
    with torch.cuda.device(device):
        check("fsdp_offload_step_units_noalloc", N.lib().fsdp_offload_step_units_noalloc(
            table, len(units), world, int(rank), dtype_code(gdt), int(bool(fp32)), dtype_code(cdt), int(chunk_numel),
            ctypes.byref(hp), int(n_threads or DEFAULT_THREADS), _stream(stream, device), _cstream(copy_stream)))
    del keep


def fsdp_offload_step_units(units, rank, fp32_reduce, hp, chunk_numel=0, n_threads=None, stream=None,
                            copy_stream=None):
    """Offloaded step of a batch of units: (OffloadState, rank_grads,
    compute_dev) triples, each state at most once; every unit's device work and
    gradient copies are enqueued first, then the host update runs over all of
    them with the copies back overlapping it."""
    device = units[0][2].device if units else None
    with torch.cuda.device(device):
        prepare_offload_step_units(units, rank, fp32_reduce, hp, chunk_numel, n_threads, stream, copy_stream)()


class OffloadState:
    """One rank's offloaded shard state for one unit: pinned host master, m, v,
    pinned staging for the gradient and compute shards, and a device buffer for
    the reduce-scatter output.  Device memory held: S elements of the gradient
    shard dtype (the fp32 state, 12 bytes per element, stays on the host), none
    with device_grad=False (for fsdp_offload_step_units_noalloc)."""

    def __init__(self, master_shard, grad_dtype, fp32_reduce, compute_dtype, device, exp_avg=None,
                 exp_avg_sq=None, device_grad=True):
        S = master_shard.numel()
        pin = dict(pin_memory=True)
        self.master = torch.empty(S, dtype=torch.float32, **pin)
        self.master.copy_(master_shard.reshape(-1).to("cpu", torch.float32))
        self.exp_avg = torch.zeros(S, dtype=torch.float32, **pin)
        self.exp_avg_sq = torch.zeros(S, dtype=torch.float32, **pin)
        if exp_avg is not None:
            self.exp_avg.copy_(exp_avg.reshape(-1).cpu())
        if exp_avg_sq is not None:
            self.exp_avg_sq.copy_(exp_avg_sq.reshape(-1).cpu())
        odt = torch.float32 if (fp32_reduce or grad_dtype == torch.float32) else grad_dtype
        self.fp32_reduce = fp32_reduce
        self.grad_dev = torch.empty(S, dtype=odt, device=device) if device_grad else None
        self.grad_host = torch.empty(S, dtype=odt, **pin)
        self.compute_host = torch.empty(S, dtype=compute_dtype, **pin)
        self.S = S

    def step(self, rank_grads, rank, hp, compute_dev, chunk_numel=0, n_threads=None, stream=None, copy_stream=None):
        return fsdp_offload_step(self.master, self.exp_avg, self.exp_avg_sq, rank_grads, rank, self.fp32_reduce,
                                 hp, self.grad_dev, self.grad_host, self.compute_host, compute_dev,
                                 chunk_numel=chunk_numel, n_threads=n_threads, stream=stream,
                                 copy_stream=copy_stream)
