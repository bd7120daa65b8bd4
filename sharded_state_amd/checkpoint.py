"""Sharded-state checkpoints of FSDP units.

"fairseq 中的 Fully Sharded Data Parallel (FSDP) 实战指南", section "工作原理"
(checkpoint paragraph): with --use-sharded-state every rank saves its own local
state to a file whose name ends in -shard{rank} and loads it back; without it
the full state is consolidated on one rank.  "FSDP (Fully Sharded Data
Parallel)", section "FSDP Checkpointing".

The file IO, checksums and staging run in libfsdp_shard.so (fsdp_save_shard,
fsdp_shard_info, fsdp_load_shard); consolidation is the library's all-gather of
the N shards followed by per-tensor views.  This module marshals arguments.
"""
import ctypes

import numpy as np
import torch

from . import _native as N
from .api import _stream, dtype_code, fsdp_unflatten_views, fsdp_unshard_gather
from ._native import AdamWHP, CkptInfo, check, i64_array

_TORCH = {N.F32: torch.float32, N.F16: torch.float16, N.BF16: torch.bfloat16}
_NP = {N.F32: np.float32, N.F16: np.uint16, N.BF16: np.uint16}


def shard_path(prefix, rank):
    """The file of rank `rank`: "<prefix>-shard<rank>"."""
    return "%s-shard%d" % (prefix, rank)


def _buf(x, name):
    """(pointer, on_device, numel, dtype code) of a torch tensor or numpy array."""
    if isinstance(x, torch.Tensor):
        if not x.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        return x.data_ptr(), int(x.device.type == "cuda"), x.numel(), dtype_code(x.dtype)
    if isinstance(x, np.ndarray):
        if not x.flags.c_contiguous:
            raise ValueError("%s must be contiguous" % name)
        code = {np.dtype(np.float32): N.F32}.get(x.dtype)
        if code is None:
            raise TypeError("%s: numpy buffers carry fp32 state (16-bit state: pass torch tensors)" % name)
        return x.ctypes.data, 0, x.size, code
    raise TypeError("%s must be a torch tensor or a numpy array" % name)


def save_shard(path, numels, world, rank, master, exp_avg, exp_avg_sq, step, hp, compute_dtype=None,
               stream=None):
    """Save one rank's shard state (master, exp_avg, exp_avg_sq: its S-element
    shards, all on the device or all on the host) of a unit with tensor sizes
    `numels`.  `step` is the number of optimizer steps taken."""
    from .api import fsdp_layout
    P, Pp, S = fsdp_layout(numels, world)
    bufs = [_buf(t, n) for t, n in ((master, "master"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"))]
    if len({(b[1], b[3]) for b in bufs}) != 1:
        raise ValueError("master, exp_avg and exp_avg_sq must share device and dtype")
    if any(b[2] != S for b in bufs):
        raise ValueError("each state buffer must hold the shard's %d elements" % S)
    if not isinstance(hp, AdamWHP):
        hp = AdamWHP(**hp)
    state = bufs[0][3]
    info = CkptInfo(world, rank, P, Pp, S, state,
                    dtype_code(compute_dtype) if compute_dtype is not None else state, int(step), hp,
                    len(numels))
    on_device = bufs[0][1]
    st = _stream(stream, master.device) if on_device else None
    check("fsdp_save_shard", N.lib().fsdp_save_shard(
        str(path).encode(), ctypes.byref(info), i64_array(numels), ctypes.c_void_p(bufs[0][0]),
        ctypes.c_void_p(bufs[1][0]), ctypes.c_void_p(bufs[2][0]), on_device, st))
    return path


def shard_info(path):
    """(header fields as a dict, tensor sizes) of a shard file."""
    info = CkptInfo()
    check("fsdp_shard_info", N.lib().fsdp_shard_info(str(path).encode(), ctypes.byref(info), None, 0))
    numels = (ctypes.c_int64 * max(info.n_tensors, 1))()
    check("fsdp_shard_info", N.lib().fsdp_shard_info(str(path).encode(), ctypes.byref(info), numels,
                                                      info.n_tensors))
    d = {k: getattr(info, k) for k, _ in CkptInfo._fields_ if k != "hp"}
    d["hp"] = AdamWHP(info.hp.lr, info.hp.beta1, info.hp.beta2, info.hp.eps, info.hp.weight_decay, info.step)
    d["state_dtype"] = _TORCH[info.state_dt]
    d["compute_dtype"] = _TORCH[info.compute_dt]
    return d, [numels[k] for k in range(info.n_tensors)]


def load_shard(path, master=None, exp_avg=None, exp_avg_sq=None, device="cuda", stream=None):
    """Load a shard file into the given buffers (allocated on `device` when
    omitted).  Returns (master, exp_avg, exp_avg_sq, header dict)."""
    info, _ = shard_info(path)
    S, sd = info["shard_numel"], info["state_dtype"]
    outs = []
    for t in (master, exp_avg, exp_avg_sq):
        outs.append(torch.empty(S, dtype=sd, device=device) if t is None else t)
    bufs = [_buf(t, "state") for t in outs]
    if len({(b[1], b[3]) for b in bufs}) != 1:
        raise ValueError("destinations must share device and dtype")
    cap = min(b[2] for b in bufs)
    on_device = bufs[0][1]
    st = _stream(stream, outs[0].device) if on_device else None
    check("fsdp_load_shard", N.lib().fsdp_load_shard(
        str(path).encode(), None, ctypes.c_void_p(bufs[0][0]), ctypes.c_void_p(bufs[1][0]),
        ctypes.c_void_p(bufs[2][0]), cap, on_device, st))
    return outs[0], outs[1], outs[2], info


def consolidate(prefix, shapes, device="cuda"):
    """The full state of a unit from its N shard files "<prefix>-shard<r>": each
    rank's master / exp_avg / exp_avg_sq shard is loaded, the N shards of each
    are gathered into the full flat buffer, and the buffer is split into
    per-tensor copies (the tail padding dropped).  Returns
    {"param": [...], "exp_avg": [...], "exp_avg_sq": [...]} plus the header."""
    info0, numels = shard_info(shard_path(prefix, 0))
    world = info0["world"]
    want = [int(np.prod(s)) for s in shapes]
    if want != numels:
        raise ValueError("shapes do not match the tensor sizes stored in the shards")
    shards = {"param": [], "exp_avg": [], "exp_avg_sq": []}
    for r in range(world):
        info, _ = shard_info(shard_path(prefix, r))
        if (info["world"], info["rank"], info["numel"]) != (world, r, info0["numel"]):
            raise ValueError("shard %d does not belong to the same unit" % r)
        p, m, v, _ = load_shard(shard_path(prefix, r), device=device)
        shards["param"].append(p)
        shards["exp_avg"].append(m)
        shards["exp_avg_sq"].append(v)
    out = {k: fsdp_unflatten_views(fsdp_unshard_gather(v), shapes, materialize=True) for k, v in shards.items()}
    out["info"] = info0
    return out
