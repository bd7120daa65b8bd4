"""Python binding of the C ABI, one function per entry point, same names.

Argument marshalling only: tensors are turned into device pointers, element
counts and the current HIP stream; every step of the pipeline runs in the HIP
kernels of libfsdp_shard.so.  PyTorch supplies device memory and streams.

Gradient, shard and full buffers are 1-D contiguous tensors on one device.
"""
import ctypes

import torch

from . import _native as N
from ._native import AdamWHP, OptimHP, Unit, View, check, i64_array, ptr_array

_DT = {torch.float32: N.F32, torch.float16: N.F16, torch.bfloat16: N.BF16}
_TORCH = {v: k for k, v in _DT.items()}


def dtype_code(dtype):
    try:
        return _DT[dtype]
    except KeyError:
        raise TypeError("unsupported dtype %s (float32, float16, bfloat16)" % dtype) from None


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor, got %s" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _same_device(tensors):
    devs = {t.device for t in tensors}
    if len(devs) > 1:
        raise ValueError("all tensors must be on one device, got %s" % sorted(map(str, devs)))


def fsdp_layout(numels, world):
    """(P, P_pad, S) of a unit with tensor sizes `numels` over `world` ranks."""
    total, padded, shard = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    check("fsdp_layout", N.lib().fsdp_layout(i64_array(numels), len(numels), int(world),
                                              ctypes.byref(total), ctypes.byref(padded),
                                              ctypes.byref(shard)))
    return total.value, padded.value, shard.value


def unit_gather_split(state_dtype, n_states, shard_elements):
    """True when a unit-step launch with a gather over `shard_elements` shard
    elements (all its units together) writes only the own slots and a second
    launch copies the peers' shards; False when the step copies them itself."""
    rc = N.lib().fsdp_unit_gather_split(dtype_code(state_dtype), int(n_states), int(shard_elements))
    if rc < 0:
        check("fsdp_unit_gather_split", rc)
    return rc == 1


def units_in_launch(world, shard_numels):
    """(units, shard elements) of the next step launch of fsdp_step_units over
    units with these shard sizes, in order: how many units it takes (0 for
    none) and how many shard elements it covers (a unit above 2^26 elements is
    stepped in 2^26-element slices, a launch each)."""
    elems = ctypes.c_int64()
    rc = N.lib().fsdp_units_in_launch(int(world), i64_array(shard_numels), len(shard_numels), ctypes.byref(elems))
    if rc < 0:
        check("fsdp_units_in_launch", rc)
    return rc, elems.value


def fsdp_flatten_pad(tensors, world, flat=None, stream=None):
    """Flatten the unit's tensors into one buffer padded with +0 to a multiple of
    `world`.  Returns the flat buffer (allocated if `flat` is None)."""
    tensors = [_dev(t, "tensors[%d]" % i) for i, t in enumerate(tensors)]
    if not tensors:
        raise ValueError("a unit needs at least one tensor")
    dt = tensors[0].dtype
    if any(t.dtype != dt for t in tensors):
        raise TypeError("all tensors of a unit must share one dtype")
    numels = [t.numel() for t in tensors]
    device = tensors[0].device
    if flat is None:   # (with `flat` given, the library call below is the only one)
        _, padded, _ = fsdp_layout(numels, world)
        flat = torch.empty(padded, dtype=dt, device=device)
    _dev(flat, "flat")
    if flat.dtype != dt:
        raise TypeError("flat dtype %s differs from the tensors' %s" % (flat.dtype, dt))
    _same_device(tensors + [flat])
    out = ctypes.c_int64()
    with torch.cuda.device(device):
        check("fsdp_flatten_pad", N.lib().fsdp_flatten_pad(
            ptr_array([t.data_ptr() for t in tensors]), i64_array(numels), len(tensors),
            dtype_code(dt), int(world), ctypes.c_void_p(flat.data_ptr()), flat.numel(),
            ctypes.byref(out), _stream(stream, device)))
    return flat[:out.value] if flat.numel() != out.value else flat


def _grads(rank_grads, shard_numel):
    rank_grads = [_dev(g, "rank_grads[%d]" % i) for i, g in enumerate(rank_grads)]
    if not rank_grads:
        raise ValueError("rank_grads is empty")
    world = len(rank_grads)
    gdt = rank_grads[0].dtype
    for i, g in enumerate(rank_grads):
        if g.dtype != gdt:
            raise TypeError("rank_grads[%d] dtype %s differs from %s" % (i, g.dtype, gdt))
        if g.numel() < world * shard_numel:
            raise ValueError("rank_grads[%d] holds %d elements, need world*shard = %d"
                             % (i, g.numel(), world * shard_numel))
    return rank_grads, world, gdt


def fsdp_reduce_scatter_local(rank_grads, rank, fp32_reduce, out=None, shard_numel=None, stream=None):
    """Rank `rank`'s averaged gradient shard from the N ranks' flat gradients.
    Output dtype: float32 if fp32_reduce or the grads are float32, else the grad dtype."""
    world = len(rank_grads)
    if shard_numel is None:
        shard_numel = rank_grads[0].numel() // world if world else 0
    rank_grads, world, gdt = _grads(rank_grads, shard_numel)
    odt = torch.float32 if (fp32_reduce or gdt == torch.float32) else gdt
    device = rank_grads[0].device
    if out is None:
        out = torch.empty(shard_numel, dtype=odt, device=device)
    _dev(out, "out")
    if out.dtype != odt or out.numel() != shard_numel:
        raise ValueError("out must be %d elements of %s" % (shard_numel, odt))
    _same_device(rank_grads + [out])
    with torch.cuda.device(device):
        check("fsdp_reduce_scatter_local", N.lib().fsdp_reduce_scatter_local(
            ptr_array([g.data_ptr() for g in rank_grads]), world, int(rank), shard_numel,
            dtype_code(gdt), int(bool(fp32_reduce)), ctypes.c_void_p(out.data_ptr()),
            _stream(stream, device)))
    return out


def fsdp_sharded_adamw(master, exp_avg, exp_avg_sq, rank_grads, rank, fp32_reduce, hp,
                       compute_shard=None, stream=None):
    """Fused reduce-scatter + AdamW + cast on rank `rank`'s shard (master, exp_avg,
    exp_avg_sq updated in place; compute_shard, if given, receives the rounded
    master).  With one already-reduced gradient shard g: rank_grads=[g], rank=0."""
    for name, t in (("master", master), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        _dev(t, name)
        if t.dtype != torch.float32:
            raise TypeError("%s must be float32" % name)
        if t.numel() != master.numel():
            raise ValueError("%s has %d elements, master %d" % (name, t.numel(), master.numel()))
    S = master.numel()
    rank_grads, world, gdt = _grads(rank_grads, S)
    tensors = rank_grads + [master, exp_avg, exp_avg_sq]
    cdt = N.F32
    cptr = None
    if compute_shard is not None:
        _dev(compute_shard, "compute_shard")
        if compute_shard.numel() != S:
            raise ValueError("compute_shard has %d elements, need %d" % (compute_shard.numel(), S))
        cdt = dtype_code(compute_shard.dtype)
        cptr = compute_shard.data_ptr()
        tensors.append(compute_shard)
    _same_device(tensors)
    if not isinstance(hp, AdamWHP):
        hp = AdamWHP(**hp)
    device = master.device
    with torch.cuda.device(device):
        check("fsdp_sharded_adamw", N.lib().fsdp_sharded_adamw(
            ctypes.c_void_p(master.data_ptr()), ctypes.c_void_p(exp_avg.data_ptr()),
            ctypes.c_void_p(exp_avg_sq.data_ptr()), ptr_array([g.data_ptr() for g in rank_grads]),
            world, int(rank), dtype_code(gdt), int(bool(fp32_reduce)), ctypes.c_void_p(cptr),
            cdt, S, ctypes.byref(hp), _stream(stream, device)))
    return compute_shard


def fsdp_step_unit(master, exp_avg, exp_avg_sq, rank_grads, rank, fp32_reduce, hp, peer_shards,
                   full, compute_shard=None, stream=None):
    """One unit's step: fused reduce-scatter + AdamW + cast of rank `rank`'s
    shard written into its slot of `full`, and the peers' compute shards
    (peer_shards[q], q != rank; entry `rank` may be None) copied into theirs --
    in the step's own launch or in a copy launch right after it, and for a
    shard above 2^26 elements slice by slice (the library's launch plan).
    compute_shard, if given, also receives this rank's compute copy."""
    for name, t in (("master", master), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        _dev(t, name)
        if t.dtype != torch.float32:
            raise TypeError("%s must be float32" % name)
        if t.numel() != master.numel():
            raise ValueError("%s has %d elements, master %d" % (name, t.numel(), master.numel()))
    S = master.numel()
    rank_grads, world, gdt = _grads(rank_grads, S)
    if len(peer_shards) != world:
        raise ValueError("peer_shards needs one entry per rank (%d), got %d" % (world, len(peer_shards)))
    _dev(full, "full")
    cdt = full.dtype
    if full.numel() != world * S:
        raise ValueError("full must hold world*shard = %d elements" % (world * S))
    tensors = rank_grads + [master, exp_avg, exp_avg_sq, full]
    ptrs = []
    for q, s in enumerate(peer_shards):
        if q == rank:
            ptrs.append(None)
            continue
        _dev(s, "peer_shards[%d]" % q)
        if s.numel() != S or s.dtype != cdt:
            raise ValueError("peer_shards[%d] must hold %d elements of %s" % (q, S, cdt))
        ptrs.append(s.data_ptr())
        tensors.append(s)
    cptr = None
    if compute_shard is not None:
        _dev(compute_shard, "compute_shard")
        if compute_shard.numel() != S or compute_shard.dtype != cdt:
            raise ValueError("compute_shard must hold %d elements of %s" % (S, cdt))
        cptr = compute_shard.data_ptr()
        tensors.append(compute_shard)
    _same_device(tensors)
    if not isinstance(hp, AdamWHP):
        hp = AdamWHP(**hp)
    device = master.device
    with torch.cuda.device(device):
        check("fsdp_step_unit", N.lib().fsdp_step_unit(
            ctypes.c_void_p(master.data_ptr()), ctypes.c_void_p(exp_avg.data_ptr()),
            ctypes.c_void_p(exp_avg_sq.data_ptr()), ptr_array([g.data_ptr() for g in rank_grads]),
            world, int(rank), dtype_code(gdt), int(bool(fp32_reduce)), ptr_array(ptrs),
            ctypes.c_void_p(full.data_ptr()), dtype_code(cdt), S, ctypes.c_void_p(cptr),
            ctypes.byref(hp), _stream(stream, device)))
    return full


def fsdp_step_units(units, rank, fp32_reduce, hp, stream=None):
    """Step several units in as few launches as possible.  `units` is a list of
    dicts with keys master, exp_avg, exp_avg_sq, rank_grads, and either
    (peer_shards, full[, compute_shard]) for the fused step with all-gather or
    compute_shard alone for the step without it.  All units share world (the
    length of rank_grads), rank, dtypes and hp.  hp is an AdamWHP (AdamW,
    fsdp_step_units) or an OptimHP (any pointwise optimizer,
    fsdp_step_units_optim; state buffers it does not keep may be None).
    Returns the prepared call after running it once, so a training loop can
    re-issue it without marshalling again: call(step=t) takes step t, and
    call.hp holds the hyper-parameters it reads (see prepare_step_units)."""
    call = prepare_step_units(units, rank, fp32_reduce, hp, stream)
    call()
    return call


def _own_hp(hp):
    """A private copy of the hyper-parameters (AdamWHP, OptimHP or an AdamWHP
    keyword dict) that a prepared call reads at every issue."""
    if isinstance(hp, (AdamWHP, OptimHP)):
        return type(hp).from_buffer_copy(hp)
    return AdamWHP(**hp)


def _reissue(fn, name, args, hp, stream, device):
    """The callable of a prepared call: call(step=None, stream=None) sets the
    step being taken (t >= 1) in its own hyper-parameters (call.hp) and issues
    the call on `stream`, else on the stream given when it was prepared, else
    on the device's current stream at the time of the call."""
    args = list(args)
    bound = _stream(stream, device) if stream is not None else None   # the null stream's handle is 0

    def call(step=None, stream=None):
        if step is not None:
            if int(step) < 1:
                raise ValueError("step must be >= 1, got %d" % int(step))
            hp.step = int(step)
        if stream is not None:
            args[-1] = _stream(stream, device)
        else:
            args[-1] = bound if bound is not None else _stream(None, device)
        with torch.cuda.device(device):
            check(name, fn(*args))

    call.hp = hp
    return call


def prepare_step_units(units, rank, fp32_reduce, hp, stream=None):
    """Marshal a fsdp_step_units call once; the returned callable issues it
    (call(step=t) for step t, call(stream=s) on stream s; see _reissue).  The
    state dtype is the dtype of the units' master tensors: float32 (fp32
    master, m, v) or bfloat16 / float16 (16-bit parameter, m, v; the parameter
    shard is the compute shard, so no compute_shard is given)."""
    if not units:
        raise ValueError("units is empty")
    optim = isinstance(hp, OptimHP)
    hp = _own_hp(hp)
    n_states = hp.n_states if optim else 2
    world = len(units[0]["rank_grads"])
    gather = units[0].get("full") is not None
    sdt = units[0]["master"].dtype
    dtype_code(sdt)
    table = (Unit * len(units))()
    keep = []
    gdt = None
    cdt = None if sdt == torch.float32 else sdt
    device = units[0]["master"].device
    tensors = []
    for k, u in enumerate(units):
        master, m, v = u["master"], u.get("exp_avg"), u.get("exp_avg_sq")
        if n_states < 2:
            v = None                              # not kept by the optimizer
        if n_states < 1:
            m = None
        for name, t in (("master", master), ("exp_avg", m), ("exp_avg_sq", v)):
            if t is None and name != "master":
                if n_states >= (1 if name == "exp_avg" else 2):
                    raise ValueError("units[%d].%s is required by the optimizer" % (k, name))
                continue
            _dev(t, "units[%d].%s" % (k, name))
            if t.dtype != sdt or t.numel() != master.numel():
                raise ValueError("units[%d].%s must be %s with master's size" % (k, name, sdt))
        S = master.numel()
        grads, w, g_dt = _grads(u["rank_grads"], S)
        if w != world:
            raise ValueError("units[%d] has %d ranks, units[0] %d" % (k, w, world))
        gdt = gdt or g_dt
        if g_dt != gdt:
            raise TypeError("every unit's gradients must share one dtype")
        full = u.get("full")
        cs = u.get("compute_shard")
        if (full is not None) != gather:
            raise ValueError("either every unit has full or none")
        if sdt != torch.float32 and cs is not None:
            raise ValueError("with 16-bit state the parameter shard is the compute shard: no compute_shard")
        out_dt = full.dtype if full is not None else (cs.dtype if cs is not None else None)
        if out_dt is not None:
            cdt = cdt or out_dt
            if out_dt != cdt:
                raise TypeError("every unit's compute dtype must be the same (and equal a 16-bit state dtype)")
        gptr = ptr_array([x.data_ptr() for x in grads])
        keep.append(gptr)
        tensors += grads + [t for t in (master, m, v) if t is not None]
        pptr = None
        if gather:
            _dev(full, "units[%d].full" % k)
            if full.numel() != world * S:
                raise ValueError("units[%d].full must hold world*shard = %d elements" % (k, world * S))
            peers = u["peer_shards"]
            if len(peers) != world:
                raise ValueError("units[%d].peer_shards needs %d entries" % (k, world))
            ptrs = []
            for q, sh in enumerate(peers):
                if q == rank:
                    ptrs.append(None)
                    continue
                _dev(sh, "units[%d].peer_shards[%d]" % (k, q))
                if sh.numel() != S or sh.dtype != full.dtype:
                    raise ValueError("units[%d].peer_shards[%d] must hold %d elements of %s" % (k, q, S, full.dtype))
                ptrs.append(sh.data_ptr())
                tensors.append(sh)
            pptr = ptr_array(ptrs)
            keep.append(pptr)
            tensors.append(full)
        if cs is not None:
            _dev(cs, "units[%d].compute_shard" % k)
            if cs.numel() != S or (cdt is not None and cs.dtype != cdt):
                raise ValueError("units[%d].compute_shard must hold %d elements of %s" % (k, S, cdt))
            tensors.append(cs)
        table[k] = Unit(master.data_ptr(), m.data_ptr() if m is not None else None,
                        v.data_ptr() if v is not None else None, gptr, pptr,
                        full.data_ptr() if full is not None else None,
                        cs.data_ptr() if cs is not None else None, S)
    _same_device(tensors)
    args = (table, len(units), world, int(rank), dtype_code(gdt), int(bool(fp32_reduce)), dtype_code(sdt),
            dtype_code(cdt or torch.float32), ctypes.byref(hp), None)
    name = "fsdp_step_units_optim" if optim else "fsdp_step_units"
    call = _reissue(getattr(N.lib(), name), name, args, hp, stream, device)
    call.keep = (keep, table, hp, tensors)   # the C side reads these host arrays at every call
    return call


def fsdp_unshard_gather(shards, full=None, stream=None):
    """Concatenate the N compute shards into the full flat buffer (a shard already
    at its slot of `full` is left in place)."""
    shards = [_dev(s, "shards[%d]" % i) for i, s in enumerate(shards)]
    if not shards:
        raise ValueError("shards is empty")
    world, S, dt = len(shards), shards[0].numel(), shards[0].dtype
    for i, s in enumerate(shards):
        if s.numel() != S or s.dtype != dt:
            raise ValueError("shards[%d] must hold %d elements of %s" % (i, S, dt))
    device = shards[0].device
    if full is None:
        full = torch.empty(world * S, dtype=dt, device=device)
    _dev(full, "full")
    if full.numel() != world * S or full.dtype != dt:
        raise ValueError("full must hold %d elements of %s" % (world * S, dt))
    _same_device(shards + [full])
    with torch.cuda.device(device):
        check("fsdp_unshard_gather", N.lib().fsdp_unshard_gather(
            ptr_array([s.data_ptr() for s in shards]), world, S, dtype_code(dt),
            ctypes.c_void_p(full.data_ptr()), _stream(stream, device)))
    return full


def fsdp_unflatten_views(full, shapes, materialize=False, stream=None):
    """Per-tensor views of the full buffer (the padding belongs to none).  With
    materialize=True each tensor is copied out into its own allocation."""
    numels = []
    for s in shapes:
        n = 1
        for x in s:
            n *= int(x)
        numels.append(n)
    views = (View * max(len(numels), 1))()
    if materialize:
        _dev(full, "full")
        outs = [torch.empty(n, dtype=full.dtype, device=full.device) for n in numels]
        with torch.cuda.device(full.device):
            check("fsdp_unflatten_views", N.lib().fsdp_unflatten_views(
                i64_array(numels), len(numels), full.numel(), views, ctypes.c_void_p(full.data_ptr()),
                dtype_code(full.dtype), ptr_array([o.data_ptr() for o in outs]),
                _stream(stream, full.device)))
        return [o.view(s) for o, s in zip(outs, shapes)]
    check("fsdp_unflatten_views", N.lib().fsdp_unflatten_views(
        i64_array(numels), len(numels), full.numel(), views, None, N.F32, None, None))
    return [full.narrow(0, views[k].offset, views[k].numel).view(shapes[k]) for k in range(len(shapes))]


def view_table(numels, padded_numel):
    """[(offset, numel)] of each tensor (host only, no device work)."""
    views = (View * max(len(numels), 1))()
    check("fsdp_unflatten_views", N.lib().fsdp_unflatten_views(
        i64_array(numels), len(numels), int(padded_numel), views, None, N.F32, None, None))
    return [(views[k].offset, views[k].numel) for k in range(len(numels))]
