"""CPU oracle for the FSDP flat-parameter shard pipeline -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library (``sharded_state_amd``)
never imports it, and it imports nothing from the product.  The arithmetic lives
in ``fsdp_oracle.c`` (plain single-threaded C); this module only moves numpy
arrays in and out of it.

Every function is pinned by the ``-m "not gpu"`` tests to something other than
itself (closed forms, invariants stated by the pages, library routines, exact
rational arithmetic, brute force on tiny inputs, the pages' printed numbers).
Throughput of the path is the only thing here that is "parity unpinned": the
pages print no number for it.

Dtype names: "f32", "f16", "bf16".  16-bit values travel as uint16 bit patterns.
"""
import ctypes
import os

import numpy as np

from . import build as _build

DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
ELEM_SIZE = {"f32": 4, "f16": 2, "bf16": 2}
NP_STORAGE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16}

_lib = None


class _HP(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("step", ctypes.c_int64)]


class _OPT(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("weight_decay", ctypes.c_float), ("momentum", ctypes.c_float),
                ("dampening", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("rho", ctypes.c_float), ("nesterov", ctypes.c_int32),
                ("step", ctypes.c_int64)]


def lib():
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        L = ctypes.CDLL(path)
        vp, i64, i32, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
        vpp = ctypes.POINTER(ctypes.c_void_p)
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_f16_to_f32.restype = ctypes.c_float
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_cast_from_f32.argtypes = [vp, ci, vp, i64]
        L.orc_cast_to_f32.argtypes = [vp, ci, vp, i64]
        L.orc_padded_numel.restype = i64
        L.orc_padded_numel.argtypes = [i64, i32]
        L.orc_offsets.argtypes = [vp, i32, vp]
        L.orc_flatten_pad.argtypes = [vpp, vp, i32, i64, i64, vp]
        L.orc_unflatten.argtypes = [vp, vp, i32, i64, vpp]
        L.orc_grad_average.argtypes = [vpp, i32, i64, i64, ci, ci, vp]
        L.orc_all_reduce.argtypes = [vpp, i32, i64, ci, ci, vp]
        L.orc_reduce_scatter.argtypes = [vpp, i32, i32, i64, ci, ci, vp]
        L.orc_adamw_scalars.argtypes = [ctypes.POINTER(_HP), vp]
        L.orc_adamw.argtypes = [vp, vp, vp, vp, i64, ctypes.POINTER(_HP)]
        L.orc_adamw16.argtypes = [vp, vp, vp, ci, vp, i64, ctypes.POINTER(_HP)]
        L.orc_cast.argtypes = [vp, ci, vp, i64]
        L.orc_sgd.argtypes = [vp, vp, vp, i64, ctypes.POINTER(_OPT)]
        L.orc_adamax.argtypes = [vp, vp, vp, vp, i64, ctypes.POINTER(_OPT)]
        L.orc_adadelta.argtypes = [vp, vp, vp, vp, i64, ctypes.POINTER(_OPT)]
        L.orc_gather.argtypes = [vpp, i32, i64, i64, vp]
        L.orc_memory_per_worker.argtypes = [i64, i32, ci, ci, ci, ctypes.c_double,
                                            ctypes.c_double, ctypes.c_double, vp]
        _lib = L
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def _ptr_array(arrs):
    return (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (np.dtype(dtype), a.dtype))
    return a


def hp(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1):
    return _HP(lr, beta1, beta2, eps, weight_decay, step)


# ---------------------------------------------------------------- formats
def f32_to(x, dt):
    """fp32 array -> storage array of dtype dt (RNE)."""
    x = _c(np.asarray(x, dtype=np.float32), np.float32)
    out = np.empty(x.shape, dtype=NP_STORAGE[dt])
    lib().orc_cast_from_f32(_ptr(x), DTYPES[dt], _ptr(out), x.size)
    return out


def to_f32(x, dt):
    """storage array of dtype dt -> fp32 (exact)."""
    x = _c(x, NP_STORAGE[dt])
    out = np.empty(x.shape, dtype=np.float32)
    lib().orc_cast_to_f32(_ptr(x), DTYPES[dt], _ptr(out), x.size)
    return out


# ---------------------------------------------------------------- layout
def padded_numel(total, world):
    return int(lib().orc_padded_numel(int(total), int(world)))


def offsets(numels):
    n = np.ascontiguousarray(np.asarray(numels, dtype=np.int64))
    out = np.empty(len(n), dtype=np.int64)
    lib().orc_offsets(_ptr(n), len(n), _ptr(out))
    return out


def flatten_pad(tensors, world, dt):
    """Concatenate 1-D views of `tensors` (storage arrays of dt) and pad with +0
    to a multiple of `world`."""
    ts = [_c(np.asarray(t).reshape(-1), NP_STORAGE[dt]) for t in tensors]
    numels = np.array([t.size for t in ts], dtype=np.int64)
    total = int(numels.sum())
    pn = padded_numel(total, world)
    flat = np.empty(pn, dtype=NP_STORAGE[dt])
    lib().orc_flatten_pad(_ptr_array(ts), _ptr(numels), len(ts), ELEM_SIZE[dt], pn, _ptr(flat))
    return flat


def unflatten(flat, shapes, dt):
    flat = _c(flat, NP_STORAGE[dt])
    numels = np.array([int(np.prod(s)) for s in shapes], dtype=np.int64)
    outs = [np.empty(int(n), dtype=NP_STORAGE[dt]) for n in numels]
    lib().orc_unflatten(_ptr(flat), _ptr(numels), len(outs), ELEM_SIZE[dt], _ptr_array(outs))
    return [o.reshape(s) for o, s in zip(outs, shapes)]


# ---------------------------------------------------------------- reduction
def _avg_dtype(grad_dt, fp32_reduce):
    return "f32" if (fp32_reduce or grad_dt == "f32") else grad_dt


def grad_average(grads, begin, count, grad_dt, fp32_reduce):
    gs = [_c(g, NP_STORAGE[grad_dt]) for g in grads]
    od = _avg_dtype(grad_dt, fp32_reduce)
    out = np.empty(count, dtype=NP_STORAGE[od])
    lib().orc_grad_average(_ptr_array(gs), len(gs), begin, count, DTYPES[grad_dt],
                           int(bool(fp32_reduce)), _ptr(out))
    return out


def all_reduce(grads, grad_dt, fp32_reduce):
    gs = [_c(g, NP_STORAGE[grad_dt]) for g in grads]
    od = _avg_dtype(grad_dt, fp32_reduce)
    out = np.empty(gs[0].size, dtype=NP_STORAGE[od])
    lib().orc_all_reduce(_ptr_array(gs), len(gs), gs[0].size, DTYPES[grad_dt],
                         int(bool(fp32_reduce)), _ptr(out))
    return out


def reduce_scatter(grads, rank, grad_dt, fp32_reduce):
    gs = [_c(g, NP_STORAGE[grad_dt]) for g in grads]
    world = len(gs)
    if gs[0].size % world:
        raise ValueError("grad length must be a multiple of the world size")
    S = gs[0].size // world
    od = _avg_dtype(grad_dt, fp32_reduce)
    out = np.empty(S, dtype=NP_STORAGE[od])
    lib().orc_reduce_scatter(_ptr_array(gs), world, rank, S, DTYPES[grad_dt],
                             int(bool(fp32_reduce)), _ptr(out))
    return out


# ---------------------------------------------------------------- optimizer
def adamw_scalars(h):
    out = np.empty(8, dtype=np.float32)
    lib().orc_adamw_scalars(ctypes.byref(h), _ptr(out))
    return out


def adamw(p, m, v, g, h):
    """In-place AdamW on fp32 arrays p, m, v with fp32 grad g."""
    for a in (p, m, v):
        if not (a.dtype == np.float32 and a.flags.c_contiguous and a.flags.writeable):
            raise TypeError("p, m, v must be writeable contiguous float32")
    g = _c(g, np.float32)
    n = p.size
    if not (m.size == n and v.size == n and g.size == n):
        raise ValueError("size mismatch")
    lib().orc_adamw(_ptr(p), _ptr(m), _ptr(v), _ptr(g), n, ctypes.byref(h))


def adamw16(p, m, v, g, h, state_dt):
    """In-place AdamW on 16-bit state (uint16 patterns of state_dt) with fp32 grad g."""
    for a in (p, m, v):
        if not (a.dtype == np.uint16 and a.flags.c_contiguous and a.flags.writeable):
            raise TypeError("p, m, v must be writeable contiguous uint16 patterns")
    g = _c(g, np.float32)
    n = p.size
    if not (m.size == n and v.size == n and g.size == n):
        raise ValueError("size mismatch")
    lib().orc_adamw16(_ptr(p), _ptr(m), _ptr(v), DTYPES[state_dt], _ptr(g), n, ctypes.byref(h))


def rank_step16(grads, rank, p_shard, m_shard, v_shard, h, grad_dt, fp32_reduce, state_dt):
    """One rank's step with 16-bit state: reduce-scatter, then AdamW on the
    16-bit parameter / m / v shard in place (the parameter is the compute copy)."""
    gshard = reduce_scatter(grads, rank, grad_dt, fp32_reduce)
    g32 = gshard if gshard.dtype == np.float32 else to_f32(gshard, grad_dt)
    adamw16(p_shard, m_shard, v_shard, g32, h, state_dt)
    return gshard


# ---------------------------------------------------------------- other pointwise optimizers
# Defaults are torch.optim's: SGD lr 1e-3 here (torch has none), Adamax lr 2e-3,
# betas (0.9, 0.999), eps 1e-8; Adadelta lr 1.0, rho 0.9, eps 1e-6.
OPT_DEFAULTS = {
    "sgd": dict(lr=1e-3, weight_decay=0.0, momentum=0.0, dampening=0.0, nesterov=False),
    "adamax": dict(lr=2e-3, weight_decay=0.0, beta1=0.9, beta2=0.999, eps=1e-8),
    "adadelta": dict(lr=1.0, weight_decay=0.0, rho=0.9, eps=1e-6),
}


def opt(kind, step=1, **kw):
    """Hyper-parameters of a pointwise optimizer ("sgd", "adamax", "adadelta")."""
    d = dict(OPT_DEFAULTS[kind])
    unknown = set(kw) - set(d)
    if unknown:
        raise TypeError("%s takes no %s" % (kind, sorted(unknown)))
    d.update(kw)
    return _OPT(d.get("lr", 0.0), d.get("weight_decay", 0.0), d.get("momentum", 0.0), d.get("dampening", 0.0),
                d.get("beta1", 0.0), d.get("beta2", 0.0), d.get("eps", 0.0), d.get("rho", 0.0),
                int(bool(d.get("nesterov", False))), int(step))


def _state(*arrs):
    for a in arrs:
        if not (a.dtype == np.float32 and a.flags.c_contiguous and a.flags.writeable):
            raise TypeError("parameter and state must be writeable contiguous float32")


def sgd(p, buf, g, o):
    """In-place SGD on fp32 p (and the momentum buffer when o.momentum != 0)."""
    _state(p)
    g = _c(g, np.float32)
    if g.size != p.size:
        raise ValueError("size mismatch")
    if o.momentum != 0.0:
        _state(buf)
        if buf.size != p.size:
            raise ValueError("size mismatch")
    lib().orc_sgd(_ptr(p), _ptr(buf) if o.momentum != 0.0 else None, _ptr(g), p.size, ctypes.byref(o))


def adamax(p, m, u, g, o):
    """In-place Adamax on fp32 p, m (first moment) and u (infinity norm)."""
    _state(p, m, u)
    g = _c(g, np.float32)
    if not (m.size == u.size == g.size == p.size):
        raise ValueError("size mismatch")
    lib().orc_adamax(_ptr(p), _ptr(m), _ptr(u), _ptr(g), p.size, ctypes.byref(o))


def adadelta(p, v, acc, g, o):
    """In-place Adadelta on fp32 p, v (squared gradients) and acc (squared updates)."""
    _state(p, v, acc)
    g = _c(g, np.float32)
    if not (v.size == acc.size == g.size == p.size):
        raise ValueError("size mismatch")
    lib().orc_adadelta(_ptr(p), _ptr(v), _ptr(acc), _ptr(g), p.size, ctypes.byref(o))


def opt_step(kind, p, s1, s2, g, o):
    """One step of optimizer `kind` ("adamw" takes an hp() as o) with state
    buffers s1, s2 in the order the library's units hold them."""
    if kind == "adamw":
        adamw(p, s1, s2, g, o)
    elif kind == "sgd":
        sgd(p, s1, g, o)
    elif kind == "adamax":
        adamax(p, s1, s2, g, o)
    elif kind == "adadelta":
        adadelta(p, s1, s2, g, o)
    else:
        raise ValueError(kind)


def rank_step_opt(kind, grads, rank, master_shard, s1, s2, o, grad_dt, fp32_reduce, compute_dt):
    """rank_step with optimizer `kind`: reduce-scatter, update in place, cast."""
    gshard = reduce_scatter(grads, rank, grad_dt, fp32_reduce)
    g32 = gshard if gshard.dtype == np.float32 else to_f32(gshard, grad_dt)
    opt_step(kind, master_shard, s1, s2, g32, o)
    return gshard, cast(master_shard, compute_dt)


def cast(master, dt):
    master = _c(master, np.float32)
    out = np.empty(master.shape, dtype=NP_STORAGE[dt])
    lib().orc_cast(_ptr(master), DTYPES[dt], _ptr(out), master.size)
    return out


def gather(shards, dt):
    ss = [_c(s, NP_STORAGE[dt]) for s in shards]
    S = ss[0].size
    if any(s.size != S for s in ss):
        raise ValueError("shards must have equal length")
    full = np.empty(S * len(ss), dtype=NP_STORAGE[dt])
    lib().orc_gather(_ptr_array(ss), len(ss), S, ELEM_SIZE[dt], _ptr(full))
    return full


def memory_per_worker(numel, world, shard_params, shard_grads, shard_optim,
                      param_bytes, grad_bytes, optim_bytes):
    """Bytes of (parameters, gradients, optimizer state) held by one worker."""
    out = np.empty(3, dtype=np.float64)
    lib().orc_memory_per_worker(int(numel), int(world), int(bool(shard_params)),
                                int(bool(shard_grads)), int(bool(shard_optim)),
                                float(param_bytes), float(grad_bytes), float(optim_bytes),
                                _ptr(out))
    return out


# ---------------------------------------------------------------- one rank's step
def rank_step(grads, rank, master_shard, m_shard, v_shard, h, grad_dt, fp32_reduce, compute_dt):
    """One rank's step of the pipeline, in the pages' order: reduce-scatter the
    N gradient buffers to this rank's averaged shard, AdamW on the fp32 shard
    (in place), cast to the compute dtype.  Returns (grad_shard, compute_shard)."""
    gshard = reduce_scatter(grads, rank, grad_dt, fp32_reduce)
    g32 = gshard if gshard.dtype == np.float32 else to_f32(gshard, grad_dt)
    adamw(master_shard, m_shard, v_shard, g32, h)
    return gshard, cast(master_shard, compute_dt)


def elementwise_step(grads_at, master, m, v, h, grad_dt, fp32_reduce, compute_dt):
    """The pipeline on a sample of elements: grads_at[q] holds rank q's gradient
    at the sampled global positions (the method is pointwise, so every output
    element depends only on the inputs at its own position).  Updates master, m,
    v in place; returns (averaged grad, compute copy)."""
    count = master.size
    avg = grad_average(grads_at, 0, count, grad_dt, fp32_reduce)
    g32 = avg if avg.dtype == np.float32 else to_f32(avg, grad_dt)
    adamw(master, m, v, g32, h)
    return avg, cast(master, compute_dt)
