#!/usr/bin/env python3
"""Benchmark of the FSDP unit pipeline on one MI355X.

Metric: GB/s and % of HBM peak for the fused reduce-scatter + AdamW + unshard
per FSDP unit.  One step = every unit slot of the workload, each through
  fused reduce-scatter + AdamW + cast (rank 0's shard)  ->  all-gather x G
  ->  per-tensor views,
on synthetic inputs already resident in HBM.  Flatten + pad is an init-time
step: it is timed separately and reported beside the line, as is the
materializing unflatten, each over independent buffer sets that together
exceed the last-level cache.

Four pipelines (--pipeline):
  units     (default) fsdp_step_units: the step of every unit of the workload
            in as few launches as the kernel-argument table allows (up to 40
            units at N <= 2, 16 at N = 8; a unit appears at most once per
            launch), each unit as in `unit`.  One launch pays the grid's
            ramp-up and drain once for all its units.
  unit      one launch per unit, fsdp_step_unit: the fused kernel writes this
            rank's compute copy straight into its slot of the full buffer and
            copies the N-1 peer shards into theirs in the same pass.  A second
            gather (reshard after forward, G = 2) reads all N shards from
            persistent compute shards, so the step also keeps a persistent
            copy of this rank's shard then.
  separate  fsdp_sharded_adamw into a compute shard, then fsdp_unshard_gather.
  offload   CPU offload of the optimizer step (fsdp_offload_step): the fp32
            master, m and v of every unit live in pinned host memory; per unit
            the device reduce-scatter, the copy of the gradient shard to the
            host, AdamW on the host cores, the copy of the compute shard back,
            then the G gathers and the views on the device.  `value` uses the
            bytes per element of `separate`, so it compares the same work;
            the "offload" object gives the host and PCIe rates it runs at.
Bytes are algorithmic, per shard element, with g and c the gradient and
compute element sizes:
  separate:     N*g (read N gradient blocks) + 12 (read master, m, v) + 12
                (write them) + c (write the compute shard) + G * 2*N*c (each
                gather reads N shards and writes N);
  unit, units:  N*g + 24 + c (own slot) + 2*(N-1)*c (peer copies)
                [+ c persistent own copy + (G-1) * 2*N*c when G = 2].
A unit pool of distinct blocks larger than the 256 MB Infinity Cache is cycled
over the slots so every step streams HBM.

Workloads (--workload): the five FSDP units of the workload table, or "all"
(the default): every one of them in this process, in the order tiny,
gpt2-large-block, gpt2-xl-model, gpt3-13b-block, llama70b-block, each with its
own roofline and CPU-oracle baseline under "configs"; the line's own fields
(value, config, roofline, cpu_baseline) are those of the largest workload that
one GPU holds, the 70B-shaped block x96 (HEADLINE).

CPU baseline: the oracle (single-threaded C) on rank 0's step of the same
units, pinned to one host core, timed over whole units -- every distinct unit
of the workload's pool once per pass, host copies of the inputs made before
the timer, state updated in place -- and reported in GB/s on the same bytes
per shard element as the GPU line.  Where the pool is smaller than the step
(the 13B and 70B workloads cycle K = 4 and K = 2 distinct blocks over 40 and
96 slots) the per-step time is the pool's extrapolated to the step, and says so.

Prints one JSON line.  --gpus above 1 exits: this measures one GPU.
"""
import argparse
import ctypes
import json
import os
import platform
import statistics
import sys
import time

HBM_PEAK_GBPS = 8000.0
METRIC = "GB/s and % HBM peak for fused reduce-scatter+AdamW+unshard per FSDP unit"
ORDER = ["tiny", "gpt2-large-block", "gpt2-xl-model", "gpt3-13b-block", "llama70b-block"]
HEADLINE = "llama70b-block"
ROOT = os.path.dirname(os.path.abspath(__file__))


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all", choices=["all"] + ORDER,
                    help="all (default: every workload, the 70B-shaped block x96 as the line's headline), or one "
                         "of " + ", ".join(ORDER))
    ap.add_argument("--pipeline", choices=["units", "unit", "separate", "offload"], default="units")
    ap.add_argument("--offload-threads", type=int, default=16,
                    help="host threads of the offloaded AdamW (--pipeline offload)")
    ap.add_argument("--offload-chunk", type=int, default=0,
                    help="elements per copy/update chunk of the offloaded step (0: the library's 4 Mi)")
    ap.add_argument("--optimizer", choices=["adamw", "sgd", "sgd-momentum", "adamax", "adadelta"], default="adamw",
                    help="pointwise optimizer of the unit step (--pipeline units; others than AdamW keep fp32 "
                         "state): SGD keeps no state, SGD with momentum one buffer, Adamax and Adadelta two")
    ap.add_argument("--state", choices=["f32", "bf16", "f16"], default="f32",
                    help="optimizer state: fp32 master/m/v (default) or 16-bit parameter/m/v with no fp32 "
                         "master (the parameter shard is the compute shard)")
    ap.add_argument("--streams", type=int, default=1,
                    help="alternate independent units over this many HIP streams (default priority), "
                         "so one unit's tail overlaps the next unit's head")
    ap.add_argument("--checkpoint", default=None, metavar="DIR",
                    help="also time saving and loading rank 0's shard state of every resident unit as "
                         "shard files in DIR (sharded-state checkpoint), reported beside the line")
    ap.add_argument("--cpu-seconds", type=float, default=2.0,
                    help="the one-core oracle baseline repeats whole passes over the workload's distinct units "
                         "until at least this long (one pass of the large workloads takes 7-20 s; 0 disables it)")
    ap.add_argument("--cpu-all-cores-seconds", type=float, default=1.0,
                    help="the same for the oracle on every host core over disjoint chunks of each unit, "
                         "reported beside the baseline (0 disables it)")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="skip the per-launch HIP events (the roofline figure needs them)")
    ap.add_argument("--event-every", type=int, default=10,
                    help="time every launch of the dominant kernel on one timed step in this many "
                         "(timing a launch costs a few microseconds of stream time)")
    ap.add_argument("--probe", choices=["copy"], default=None,
                    help="copy: time a plain 1 GiB copy with the gather kernel (counter calibration)")
    return ap.parse_args()


def sizes(cfg, pipeline, state="f32", n_states=2, split=False):
    """(dominant kernel bytes, whole-step bytes) per shard element; the
    parameter and each of the optimizer's n_states state buffers are read and
    written.  Unit step: the kernel writes the own slot, and copies the N-1
    peers' shards in its trip unless `split` (the library's launch plan,
    unit_gather_split) leaves them to a launch of their own."""
    g = 4 if cfg.grad_dt == "f32" else 2
    c = 4 if cfg.compute_dt == "f32" else 2
    N, G = cfg.world, cfg.gathers
    if state != "f32":               # 16-bit parameter, m, v; the parameter is the compute copy
        kernel = N * g + 12 + c
        step = kernel + 2 * (N - 1) * c + (G - 1) * 2 * N * c
        return (kernel if split else kernel + 2 * (N - 1) * c), step
    st = 8 * (1 + n_states)
    if pipeline == "separate":
        fused = N * g + st + c
        return fused, fused + G * 2 * N * c
    kernel = N * g + st + c + (c if G > 1 else 0)
    step = kernel + 2 * (N - 1) * c + (G - 1) * 2 * N * c
    return (kernel if split else kernel + 2 * (N - 1) * c), step


def optimizer_hp(name, cfg, N):
    """Hyper-parameters of --optimizer (AdamW: the workload's)."""
    if name == "adamw":
        return None
    return {"sgd": N.OptimHP.sgd(lr=1e-2, weight_decay=1e-4),
            "sgd-momentum": N.OptimHP.sgd(lr=1e-2, momentum=0.9, weight_decay=1e-4),
            "adamax": N.OptimHP.adamax(weight_decay=0.01),
            "adadelta": N.OptimHP.adadelta(weight_decay=0.01)}[name].at_step(cfg.step)


class Unit:
    """Rank 0's resident buffers for one distinct block of the pool."""

    def __init__(self, cfg, block, ss, torch, workloads, state="f32"):
        dev = "cuda"
        P, Pp, S = ss.fsdp_layout(cfg.numels, cfg.world)
        self.P, self.Pp, self.S = P, Pp, S
        sd = workloads.TORCH_DTYPE[state]
        params = workloads.param_tensors(cfg, block, dev)
        if state != "f32":
            params = [t.to(sd) for t in params]
        flat = ss.fsdp_flatten_pad(params, cfg.world)
        del params
        # the N ranks' gradients as the rows of one buffer (workloads.rank_grads)
        self.grads = list(workloads.rank_grads(cfg, block, Pp, dev).unbind(0))
        cdt = workloads.TORCH_DTYPE[cfg.compute_dt] if state == "f32" else sd
        hp = ss.AdamWHP(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.step)
        # peers' compute shards: the other ranks' own steps on the same unit
        self.peers = []
        for q in range(1, cfg.world):
            mq, vq = (x.to(sd) for x in workloads.moments(cfg, block, q * S, S, P, dev))
            pq = flat[q * S:(q + 1) * S].clone()
            if state == "f32":
                # reduce-scatter, then the step on the reduced shard (same bytes as the fused
                # form; its one-rank kernel keeps set-up launches apart from the timed ones
                # in profiles)
                cq = torch.empty(S, dtype=cdt, device=dev)
                gq = ss.fsdp_reduce_scatter_local(self.grads, q, cfg.fp32_reduce)
                ss.fsdp_sharded_adamw(pq, mq, vq, [gq], 0, cfg.fp32_reduce, hp, compute_shard=cq)
                del gq
            else:
                ss.fsdp_step_units([dict(master=pq, exp_avg=mq, exp_avg_sq=vq, rank_grads=self.grads)], q,
                                   cfg.fp32_reduce, hp)
                cq = pq
            self.peers.append(cq)
            del mq, vq
        self.master = flat[:S].clone()
        del flat
        self.m, self.v = (x.to(sd) for x in workloads.moments(cfg, block, 0, S, P, dev))
        self.compute = torch.empty(S, dtype=cdt, device=dev) if state == "f32" else self.master
        self.full = torch.empty(Pp, dtype=cdt, device=dev)
        torch.cuda.synchronize()


SEG_PER_LAUNCH = 64   # segments (tensors + zero tail) per flatten launch


# Bytes that one rotation of the flatten / unflatten rate measurements touches
# at least: four times the 256 MB last-level (Infinity) cache, so that a call's
# buffers have been evicted before the rotation comes back to them and each call
# streams HBM.
ROTATION_BYTES = 4 * (256 << 20)
ROTATION_MAX = 64


def rotation(nbytes):
    """Number of independent buffer sets for a call that moves `nbytes` bytes."""
    return max(1, min(ROTATION_MAX, -(-ROTATION_BYTES // max(1, nbytes))))


def call_ms(fn, name, calls, launches, torch, N, lib, reps=5):
    """Mean device time of one C-ABI call over max(reps, len(calls)) calls after
    two warm-up calls, rotating over `calls` (argument tuples marshalled once,
    each on its own buffers): events on the kernel's own dispatch when the call
    makes one launch, else two stream events around the calls back to back."""
    reps = max(reps, len(calls))
    for r in range(2):
        N.check(name, fn(*calls[r % len(calls)]))
    torch.cuda.synchronize()
    if launches == 1:   # events on the kernel's dispatch packet
        evs = HipEvents(2 * reps)
        for r in range(reps):
            N.check("fsdp_time_next_launch", lib.fsdp_time_next_launch(evs.ev[2 * r], evs.ev[2 * r + 1]))
            N.check(name, fn(*calls[r % len(calls)]))
        torch.cuda.synchronize()
        ms = statistics.fmean([evs.elapsed_ms(2 * r, 2 * r + 1) for r in range(reps)])
        evs.close()
    else:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(reps):
            N.check(name, fn(*calls[r % len(calls)]))
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
    return ms


def flatten_rate(cfg, ss, torch, N, lib, workloads, state="f32", reps=5):
    """fsdp_flatten_pad of the first block's tensors into a preallocated flat
    buffer, called through the C ABI (marshalled once per buffer set): mean
    kernel duration over the calls of a rotation over independent copies of the
    tensors and the flat buffer (rotation(): at least 1 GB per rotation), after
    two warm-up calls, and the rate of its bytes (read P, write the padded
    length)."""
    params = workloads.param_tensors(cfg, 0, "cuda")
    if state != "f32":
        params = [t.to(workloads.TORCH_DTYPE[state]) for t in params]
    P, Pp, _ = ss.fsdp_layout(cfg.numels, cfg.world)
    es = params[0].element_size()
    nbytes = P * es + Pp * es
    sets = [(params, torch.empty(Pp, dtype=params[0].dtype, device="cuda"))]
    for _ in range(rotation(nbytes) - 1):
        sets.append(([t.clone() for t in params], torch.empty(Pp, dtype=params[0].dtype, device="cuda")))
    padded = ctypes.c_int64()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    calls = [(N.ptr_array([t.data_ptr() for t in ps]), N.i64_array(cfg.numels), len(cfg.numels),
              ss.dtype_code(flat.dtype), cfg.world, ctypes.c_void_p(flat.data_ptr()), flat.numel(),
              ctypes.byref(padded), stream) for ps, flat in sets]
    segs = sum(1 for n in cfg.numels if n > 0) + (1 if Pp > P else 0)
    launches = (segs + SEG_PER_LAUNCH - 1) // SEG_PER_LAUNCH
    ms = call_ms(lib.fsdp_flatten_pad, "fsdp_flatten_pad", calls, launches, torch, N, lib, reps)
    del params, sets, calls
    return {"avg_ms": round(ms, 4), "bytes": nbytes, "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "tensors": len(cfg.numels), "launches": launches, "buffer_sets": rotation(nbytes)}


def unflatten_rate(cfg, ss, torch, N, lib, workloads, state="f32", reps=5):
    """fsdp_unflatten_views materializing the first block's tensors out of a
    gathered full buffer of the compute dtype into preallocated per-tensor
    destinations, called through the C ABI, timed as the flatten (a rotation
    over independent full buffers and destinations); bytes: P elements read and
    P written (the padding is no view)."""
    cdt = workloads.TORCH_DTYPE[cfg.compute_dt if state == "f32" else state]
    P, Pp, _ = ss.fsdp_layout(cfg.numels, cfg.world)
    es = torch.empty(0, dtype=cdt).element_size()
    nbytes = 2 * P * es
    views = (N.View * len(cfg.numels))()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sets, calls = [], []
    for _ in range(rotation(nbytes)):
        full = torch.empty(Pp, dtype=cdt, device="cuda")
        full.view(torch.uint8).fill_(0x3c)
        dsts = [torch.empty(n, dtype=cdt, device="cuda") for n in cfg.numels]
        sets.append((full, dsts))
        calls.append((N.i64_array(cfg.numels), len(cfg.numels), Pp, views, ctypes.c_void_p(full.data_ptr()),
                      ss.dtype_code(cdt), N.ptr_array([d.data_ptr() for d in dsts]), stream))
    segs = sum(1 for n in cfg.numels if n > 0)
    launches = (segs + SEG_PER_LAUNCH - 1) // SEG_PER_LAUNCH
    ms = call_ms(lib.fsdp_unflatten_views, "fsdp_unflatten_views", calls, launches, torch, N, lib, reps)
    del sets, calls
    return {"avg_ms": round(ms, 4), "bytes": nbytes, "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "tensors": len(cfg.numels), "launches": launches, "dtype": str(cdt).replace("torch.", ""),
            "buffer_sets": rotation(nbytes)}


def cpu_host_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.machine()


class HostUnit:
    """Host copies of rank 0's inputs of one unit, made before any timing:
    block 0 of each rank's gradient, the parameter/state shards (updated in
    place by the oracle) and the peers' compute shards."""

    def __init__(self, unit, np_of_bytes):
        S = unit.S
        self.S = S
        self.grads = [np_of_bytes(x[:S]).copy() for x in unit.grads]
        self.peers = [np_of_bytes(q).copy() for q in unit.peers]
        self.p, self.m, self.v = (np_of_bytes(t).copy() for t in (unit.master, unit.m, unit.v))


def cpu_baseline(cfg, hosts, per_elt, state="f32", ohp=None, threads=1, min_seconds=0.0, blocks=None):
    """The oracle on rank 0's step of every unit in `hosts` (HostUnit), in
    unit order: reduce-scatter, the optimizer step in place, cast, and the
    workload's G gathers.  One pass covers every unit once; passes repeat until
    `min_seconds` (at least one).  threads == 1: on one pinned host core;
    otherwise on `threads` Python threads over disjoint chunks of each unit
    (the oracle's C calls run outside the GIL).  GB/s counts `per_elt` bytes per
    shard element, the GPU line's count.  With `blocks` (> len(hosts)) slots
    per step, the per-step time is the pass time scaled to the step."""
    import numpy as np
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    h = oracle.hp(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.step)
    opt = oracle_opt(oracle, ohp) if ohp is not None else None
    cdt = cfg.compute_dt if state == "f32" else state

    def step(u, lo, n):
        avg = oracle.grad_average(u.grads, lo, n, cfg.grad_dt, cfg.fp32_reduce)
        g32 = avg if avg.dtype == np.float32 else oracle.to_f32(avg, cfg.grad_dt)
        p, m, v = u.p[lo:lo + n], u.m[lo:lo + n], u.v[lo:lo + n]
        if opt is not None:
            oracle.opt_step(opt[0], p, m, v, g32, opt[1])
            comp = oracle.cast(p, cfg.compute_dt)
        elif state == "f32":
            oracle.adamw(p, m, v, g32, h)
            comp = oracle.cast(p, cfg.compute_dt)
        else:
            oracle.adamw16(p, m, v, g32, h, state)
            comp = p
        for _ in range(cfg.gathers):
            oracle.gather([comp] + [q[lo:lo + n] for q in u.peers], cdt)

    items = []
    for u in hosts:
        parts = threads if threads > 1 else 1
        bounds = [u.S * k // parts for k in range(parts + 1)]
        items += [(u, a, b - a) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    elems_per_pass = sum(u.S for u in hosts)
    cores_before = None
    if threads == 1:
        try:
            cores_before = os.sched_getaffinity(0)
            os.sched_setaffinity(0, {sorted(cores_before)[0]})
        except (AttributeError, OSError):
            cores_before = None
    passes = 0
    ex = ThreadPoolExecutor(threads) if threads > 1 else None
    try:
        t0 = time.perf_counter()
        while True:
            if ex is None:
                for it in items:
                    step(*it)
            else:
                list(ex.map(lambda it: step(*it), items))
            passes += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
        dt = time.perf_counter() - t0
    finally:
        if ex is not None:
            ex.shutdown()
        if cores_before is not None:
            os.sched_setaffinity(0, cores_before)
    eps = passes * elems_per_pass / dt
    pass_s = dt / passes
    opt_name = ohp.name if ohp is not None else ("AdamW" if state == "f32" else "AdamW on %s state" % state)
    where = ("one pinned core" if threads == 1 else
             "%d threads over %d disjoint chunks of each unit" % (threads, threads))
    extrap = blocks is not None and blocks > len(hosts)
    if extrap:
        what = ("the K = %d distinct blocks of the pool (%d shard elements), extrapolated from K = %d to the "
                "%d-block step" % (len(hosts), elems_per_pass, len(hosts), blocks))
        step_s = pass_s * blocks / len(hosts)
    else:
        what = ("whole units: all %d block%s of the step (%d shard elements)"
                % (len(hosts), "s" if len(hosts) > 1 else "", elems_per_pass))
        step_s = pass_s
    return {
        "value": round(eps * per_elt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": "rank 0's step (reduce-scatter, %s, cast, %d gather%s) on %s, on %s; %d pass%s in %.1f s; "
                  "%d B per shard element as the GPU line; host copies made before the timer; host %s (%s cpus)"
                  % (opt_name, cfg.gathers, "s" if cfg.gathers > 1 else "", what, where, passes,
                     "es" if passes > 1 else "", dt, per_elt, cpu_host_model(), os.cpu_count()),
        "elements_per_s": round(eps, 1),
        "bytes_per_shard_element": per_elt,
        "seconds_per_step": round(step_s, 4),
        "extrapolated": bool(extrap),
    }


def oracle_opt(oracle, hp):
    """(kind, oracle hyper-parameters) of an OptimHP, for opt_step(kind, p, s1, s2, g, o)."""
    if hp.kind == 1:
        o = oracle.opt("sgd", step=hp.step, lr=hp.lr, weight_decay=hp.weight_decay, momentum=hp.momentum,
                       dampening=hp.dampening, nesterov=bool(hp.nesterov))
        return "sgd", o
    if hp.kind == 2:
        return "adamax", oracle.opt("adamax", step=hp.step, lr=hp.lr, weight_decay=hp.weight_decay,
                                    beta1=hp.beta1, beta2=hp.beta2, eps=hp.eps)
    return "adadelta", oracle.opt("adadelta", step=hp.step, lr=hp.lr, weight_decay=hp.weight_decay, rho=hp.rho,
                                  eps=hp.eps)


class HipEvents:
    """Pre-created HIP events recorded with direct hipEventRecord calls on the
    launch stream (no per-record allocation or wrapper work)."""

    def __init__(self, count):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(count):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e)
        self.record = self.hip.hipEventRecord

    def elapsed_ms(self, i, j):
        out = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[i], self.ev[j])
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (hipError_t %d)" % rc)
        return out.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def traffic_from_profiles(kernel_tag, src_hash):
    """Counter-measured HBM bytes per launch, if a summary for this exact kernel
    source is committed under profiles/."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.txt" % kernel_tag)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != src_hash:
        return None
    try:
        return float(vals["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


KERNEL_SOURCES = ("fsdp_kernels.hip", "fsdp_kernels.h", "fsdp_device.h", "fsdp_units.h", "fsdp_optim.h",
                  "fsdp_units_adamw.hip", "fsdp_units_sgd.hip", "fsdp_units_adamax.hip", "fsdp_units_adadelta.hip")


def kernel_code(text):
    """A device source with its comments and blank lines removed (the sources
    hold no comment markers inside string literals)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash():
    """sha256 over the device sources' code (comments excluded), so counter
    figures taken on another version of the kernels are not reported."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        src = open(os.path.join(ROOT, "sharded_state_amd", "csrc", f), encoding="utf-8").read()
        h.update(kernel_code(src).encode())
    return h.hexdigest()


def copy_ceiling(torch, N, lib, reps=20):
    """Achievable HBM rate of a plain copy: 1 GiB through the library's gather
    kernel (one shard), the ceiling a read+write stream reaches on this machine."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    copy = (N.ptr_array([a.data_ptr()]), 1, n // 4, N.F32, ctypes.c_void_p(b.data_ptr()), st)
    for _ in range(3):
        N.check("fsdp_unshard_gather", lib.fsdp_unshard_gather(*copy))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        lib.fsdp_unshard_gather(*copy)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    torch.cuda.empty_cache()
    return {"bytes_read": n, "bytes_written": n, "ms": round(ms, 5), "gbps": round(2 * n / ms / 1e6, 1)}


def bench_offload(args, cfg, torch, ss, N, workloads):
    """--pipeline offload: the step of every unit slot with its optimizer state
    in pinned host memory (fsdp_offload_step_units over batches of distinct
    units), then the device gathers."""
    _, per_elt = sizes(cfg, "separate")
    pool = [Unit(cfg, b, ss, torch, workloads) for b in range(cfg.pool)]
    S = pool[0].S
    cdt = pool[0].compute.dtype
    threads = max(1, args.offload_threads)
    states = []
    for u in pool:
        states.append(ss.OffloadState(u.master, u.grads[0].dtype, cfg.fp32_reduce, cdt, "cuda",
                                      exp_avg=u.m, exp_avg_sq=u.v))
        del u.master, u.m, u.v                  # the fp32 state lives on the host only
    torch.cuda.empty_cache()
    hp = ss.AdamWHP(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.step)
    G = cfg.gathers
    slots = [k % len(pool) for k in range(cfg.blocks)]
    shard_lists = [[u.compute] + u.peers for u in pool]
    # batches of distinct units; the copies back and the gathers of a batch run
    # on a second stream, so the next batch's reduce-scatter and copies to the
    # host do not queue behind them
    copy_stream = torch.cuda.Stream()
    nb = -(-len(slots) // len(pool))
    bounds = [round(j * len(slots) / nb) for j in range(nb + 1)]
    batches = []
    for j in range(nb):
        ids = slots[bounds[j]:bounds[j + 1]]
        call = ss.prepare_offload_step_units([(states[i], pool[i].grads, pool[i].compute) for i in ids], 0,
                                             cfg.fp32_reduce, hp, chunk_numel=args.offload_chunk,
                                             n_threads=threads, copy_stream=copy_stream)
        batches.append((call, ids))

    def step():
        for call, ids in batches:
            call()
            with torch.cuda.stream(copy_stream):
                for i in ids:
                    for _ in range(G):
                        ss.fsdp_unshard_gather(shard_lists[i], full=pool[i].full)
                    ss.fsdp_unflatten_views(pool[i].full, cfg.shapes)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    gbps = per_elt * S * cfg.blocks / (ms_step * 1e-3) / 1e9

    # the parts alone, on unit 0: host AdamW, device-to-host and host-to-device copies
    st, u = states[0], pool[0]
    gsz, csz = st.grad_host.element_size(), st.compute_host.element_size()
    host_b = S * (12 + gsz + 12 + csz)            # read master, m, v, grad; write master, m, v, compute
    reps = 5
    t = time.perf_counter()
    for _ in range(reps):
        ss.fsdp_host_adamw(st.master, st.exp_avg, st.exp_avg_sq, st.grad_host, hp, compute=st.compute_host,
                           n_threads=threads)
    host_s = (time.perf_counter() - t) / reps
    t = time.perf_counter()
    ss.fsdp_host_adamw(st.master, st.exp_avg, st.exp_avg_sq, st.grad_host, hp, compute=st.compute_host,
                       n_threads=1)
    host1_s = time.perf_counter() - t

    def copy_rate(dst, src):
        dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(reps):
            dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        return src.numel() * src.element_size() * reps / (time.perf_counter() - t) / 1e9

    # host memory rates on the same cores: a threaded copy and two threaded
    # read-only passes of 2 GiB (torch's sum, and numpy sums of `threads`
    # slices on as many Python threads, which numpy runs outside the GIL), the
    # best of 7 passes each
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    a = torch.ones(1 << 29, dtype=torch.float32)
    b = torch.empty_like(a)
    b.copy_(a)
    a.sum()
    words = a.numpy().view(np.uint64)
    host_copy = host_read = 0.0
    for workers in sorted({max(1, threads // 2), threads}):
        slices = np.array_split(words, workers)
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(np.bitwise_or.reduce, slices))
            for _ in range(7):
                t = time.perf_counter()
                b.copy_(a)
                host_copy = max(host_copy, 2 * a.numel() * 4 / (time.perf_counter() - t) / 1e9)
                t = time.perf_counter()
                a.sum()
                host_read = max(host_read, a.numel() * 4 / (time.perf_counter() - t) / 1e9)
                t = time.perf_counter()
                list(ex.map(np.bitwise_or.reduce, slices))
                host_read = max(host_read, a.numel() * 4 / (time.perf_counter() - t) / 1e9)
    del a, b, words, slices
    d2h = copy_rate(st.grad_host, st.grad_dev)
    h2d = copy_rate(u.compute, st.compute_host)
    pcie_b = S * (gsz + csz)
    off = {
        "threads": threads, "chunk_numel": args.offload_chunk or 4 << 20, "units_per_call": len(batches[0][1]),
        "host_copy_gbps": round(host_copy, 2), "host_read_gbps": round(host_read, 2),
        "torch_cpu_threads": torch.get_num_threads(),
        "host_state_bytes_per_unit": 12 * S, "device_state_bytes_per_unit": 0,
        "host_adamw_bytes_per_element": 12 + gsz + 12 + csz,
        "host_adamw_gbps": round(host_b / host_s / 1e9, 2),
        "host_adamw_ms_per_unit": round(host_s * 1e3, 3),
        "host_adamw_1thread_gbps": round(host_b / host1_s / 1e9, 2),
        "pcie_bytes_per_element": gsz + csz,
        "d2h_copy_gbps": round(d2h, 2), "h2d_copy_gbps": round(h2d, 2),
        "step_host_gbps": round(host_b * cfg.blocks / (ms_step * 1e-3) / 1e9, 2),
        "step_host_gbps_with_dma": round((host_b + pcie_b) * cfg.blocks / (ms_step * 1e-3) / 1e9, 2),
        "step_pcie_gbps": round(pcie_b * cfg.blocks / (ms_step * 1e-3) / 1e9, 2),
    }
    # the bound of the offloaded step is host DRAM: the host AdamW's own bytes
    # per step time, against the best threaded read-only rate of the same cores
    # measured in this run (no published figure for this host); the copies'
    # DMA through host memory is reported beside it (step_host_gbps_with_dma).
    # The read probes are library reductions and can fall below the host
    # kernel's own rate; then no peak and no fraction are claimed.
    ach = off["step_host_gbps"]
    probe = off["host_read_gbps"]
    roof = {"bound": "host", "achieved": ach, "peak": probe if probe >= ach else None, "unit": "GB/s",
            "frac": round(ach / probe, 4) if probe >= ach else None, "traffic": None,
            "kernel": "fsdp_host_adamw (%d threads) inside the offloaded step; peak = best threaded host read "
                      "rate measured in this run (torch sum, numpy OR-reductions on threads), none when that "
                      "probe reaches less than the achieved rate" % threads,
            "read_probe_gbps": probe}
    out = {
        "metric": METRIC, "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "%s x%d" % (cfg.name, cfg.blocks), "pipeline": "offload", "state_dtype": "f32",
                   "world": cfg.world, "rank": 0, "shard_numel": S, "blocks_per_step": cfg.blocks,
                   "distinct_blocks": cfg.pool, "grad_dtype": cfg.grad_dt,
                   "fp32_reduce_scatter": cfg.fp32_reduce, "compute_dtype": cfg.compute_dt,
                   "gathers_per_step": G, "bytes_per_shard_element": per_elt},
        "shard_elements_per_s": round(S * cfg.blocks / (ms_step * 1e-3), 1),
        "roofline": roof, "offload": off, "cpu_baseline": None,
    }
    return out


def run_workload(args, cfg, torch, ss, N, lib, workloads):
    """One workload: set-up, warm-up, K timed steps, the roofline of the
    dominant launch, the CPU-oracle baselines and the flatten and unflatten rates."""
    if args.pipeline == "offload":
        return bench_offload(args, cfg, torch, ss, N, workloads)
    ohp = optimizer_hp(args.optimizer, cfg, N)
    n_states = ohp.n_states if ohp is not None else 2
    fused_b, per_elt = sizes(cfg, "separate" if args.pipeline == "separate" else "unit", args.state, n_states)
    pool = [Unit(cfg, b, ss, torch, workloads, args.state) for b in range(cfg.pool)]
    S = pool[0].S
    stream = torch.cuda.current_stream()
    streams = [stream] + [torch.cuda.Stream() for _ in range(max(1, args.streams) - 1)]
    st_handles = [ctypes.c_void_p(x.cuda_stream) for x in streams]
    hp = ss.AdamWHP(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.step)
    hp_ref = ctypes.byref(hp)
    gcode, ccode = ss.dtype_code(pool[0].grads[0].dtype), ss.dtype_code(pool[0].compute.dtype)
    scode = ss.dtype_code(pool[0].master.dtype)
    state16 = args.state != "f32"
    numels = N.i64_array(cfg.numels)
    views = (N.View * len(cfg.numels))()

    # prepared ctypes arguments: marshalling happens once, outside the timed region
    unit_pipe = args.pipeline in ("unit", "units")
    G = cfg.gathers
    per_unit = []
    for i, u in enumerate(pool):
        grads = N.ptr_array([x.data_ptr() for x in u.grads])
        p, m, v = (ctypes.c_void_p(t.data_ptr()) for t in (u.master, u.m, u.v))
        shards = N.ptr_array([u.compute.data_ptr()] + [q.data_ptr() for q in u.peers])
        peer_tab = N.ptr_array([0] + [q.data_ptr() for q in u.peers])
        full = ctypes.c_void_p(u.full.data_ptr())
        persistent = u.compute.data_ptr() if (G > 1 and not state16) else None
        desc = N.Unit(u.master.data_ptr(), u.m.data_ptr() if n_states >= 1 else None,
                      u.v.data_ptr() if n_states >= 2 else None, grads, peer_tab, u.full.data_ptr(), persistent, S)
        unflat = (numels, len(cfg.numels), u.Pp, views, None, ccode, None, None)
        per_unit.append(dict(grads=grads, p=p, m=m, v=v, shards=shards, peer_tab=peer_tab, full=full,
                             persistent=ctypes.c_void_p(persistent), desc=desc, views=unflat))

    # launch groups: (first call, units in it, trailing calls), in slot order
    slots = [k % len(pool) for k in range(cfg.blocks)]
    groups = []
    if args.pipeline == "units":
        # one call per step launch, packed as the library packs (units_in_launch);
        # a unit appears at most once per launch
        lim = min(ss.units_in_launch(cfg.world, [S] * len(pool))[0], len(pool))
        nb = -(-len(slots) // lim)
        bounds = [round(j * len(slots) / nb) for j in range(nb + 1)]
        for j in range(nb):
            batch = slots[bounds[j]:bounds[j + 1]]
            st = st_handles[j % len(st_handles)]
            table = (N.Unit * len(batch))(*[per_unit[i]["desc"] for i in batch])
            if ohp is None:
                first = (lib.fsdp_step_units, (table, len(batch), cfg.world, 0, gcode, int(cfg.fp32_reduce), scode,
                                               ccode, hp_ref, st))
            else:
                first = (lib.fsdp_step_units_optim, (table, len(batch), cfg.world, 0, gcode, int(cfg.fp32_reduce),
                                                     scode, ccode, ctypes.byref(ohp), st))
            trail = [(lib.fsdp_unshard_gather, (per_unit[i]["shards"], cfg.world, S, ccode, per_unit[i]["full"], st))
                     for i in batch for _ in range(G - 1)]
            trail += [(lib.fsdp_unflatten_views, per_unit[i]["views"]) for i in batch]
            groups.append((first, len(batch), trail, table))
    else:
        for j, i in enumerate(slots):
            d = per_unit[i]
            st = st_handles[j % len(st_handles)] if args.streams > 1 else st_handles[0]
            if args.pipeline == "unit" and state16:
                table = (N.Unit * 1)(d["desc"])
                first = (lib.fsdp_step_units, (table, 1, cfg.world, 0, gcode, int(cfg.fp32_reduce), scode, ccode,
                                               hp_ref, st))
                d["table"] = table
                trail = [(lib.fsdp_unshard_gather, (d["shards"], cfg.world, S, ccode, d["full"], st))] * (G - 1)
            elif args.pipeline == "unit":
                first = (lib.fsdp_step_unit, (d["p"], d["m"], d["v"], d["grads"], cfg.world, 0, gcode,
                                              int(cfg.fp32_reduce), d["peer_tab"], d["full"], ccode, S,
                                              d["persistent"], hp_ref, st))
                trail = [(lib.fsdp_unshard_gather, (d["shards"], cfg.world, S, ccode, d["full"], st))] * (G - 1)
            else:
                first = (lib.fsdp_sharded_adamw, (d["p"], d["m"], d["v"], d["grads"], cfg.world, 0, gcode,
                                                  int(cfg.fp32_reduce), ctypes.c_void_p(pool[i].compute.data_ptr()),
                                                  ccode, S, hp_ref, st))
                trail = [(lib.fsdp_unshard_gather, (d["shards"], cfg.world, S, ccode, d["full"], st))] * G
            trail = trail + [(lib.fsdp_unflatten_views, d["views"])]
            groups.append((first, 1, trail, None))
    # Per-launch timing: the library attaches a start/stop event pair to the
    # dominant kernel's own dispatch packet (fsdp_time_next_launch), so the
    # timed region carries no extra stream packets.
    use_events = not args.no_kernel_events
    nslot = len(groups)
    every = max(1, args.event_every)
    ev_steps = [k for k in range(args.steps) if k % every == 0] if use_events else []
    evs = HipEvents(2 * nslot * len(ev_steps)) if use_events else None
    arm = lib.fsdp_time_next_launch

    def step(ev_base=None):
        for i, ((f0, a0), _, trail, _) in enumerate(groups):
            if ev_base is not None:
                arm(evs.ev[2 * (ev_base + i)], evs.ev[2 * (ev_base + i) + 1])
            rc = f0(*a0)
            if rc:
                N.check(f0.__name__, rc)
            for fg, ag in trail:
                rc = fg(*ag)
                if rc:
                    N.check(fg.__name__, rc)

    def fork():
        for x in streams[1:]:
            x.wait_stream(stream)

    def join():
        for x in streams[1:]:
            stream.wait_stream(x)

    fork()
    for _ in range(args.warmup):
        step()
    join()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    fork()
    for k in range(args.steps):
        step((k // every) * nslot if (use_events and k % every == 0) else None)
    join()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    ms_step = total_ms / args.steps
    bytes_step = per_elt * S * cfg.blocks
    gbps = bytes_step / (ms_step * 1e-3) / 1e9

    roof = None
    if use_events:
        durs = [evs.elapsed_ms(2 * k, 2 * k + 1) for k in range(nslot * len(ev_steps))]
        evs.close()
        avg_ms = statistics.fmean(durs)
        # the timed launch is the first of each call: the library's plan says how
        # many units it takes and how many shard elements it covers (a unit above
        # 2^26 elements is stepped in 2^26-element slices, a launch each)
        plan_units, launch_elems = ss.units_in_launch(cfg.world, [S] * groups[0][1])
        split = unit_pipe and ss.unit_gather_split(pool[0].master.dtype, n_states, launch_elems)
        fused_b, _ = sizes(cfg, "separate" if args.pipeline == "separate" else "unit", args.state, n_states,
                           split)
        bytes_per_launch = fused_b * launch_elems
        per_launch = ("%d units per launch" % plan_units if launch_elems == plan_units * S else
                      "one %d-element slice of a unit per launch" % launch_elems)
        achieved = bytes_per_launch / (avg_ms * 1e-3) / 1e9
        tag = args.pipeline if args.optimizer == "adamw" else "%s-%s" % (args.pipeline, args.optimizer)
        if args.state != "f32":
            tag += "-state-" + args.state          # another kernel: counters of its own
        traffic = traffic_from_profiles("%s_%s" % (tag, cfg.name), kernel_source_hash())
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": (("k_units<GATHER> (fused reduce-scatter + optimizer + cast + all-gather, %s)"
                            if not split else
                            "k_units (fused reduce-scatter + optimizer + cast + own-slot write, %s; the peers' "
                            "slots follow in one batched copy launch)") % per_launch
                           if unit_pipe else "k_units (fused reduce-scatter + optimizer + cast, %s)" % per_launch),
                "shard_elements_per_launch": int(launch_elems),
                "peer_copies_in_own_launch": bool(split),
                "bytes_per_launch": int(bytes_per_launch), "avg_launch_ms": round(avg_ms, 5),
                "timed_launches": len(durs),
                "median_launch_ms": round(statistics.median(durs), 5),
                "min_launch_ms": round(min(durs), 5), "max_launch_ms": round(max(durs), 5)}

    cpu = cpu_all = None
    if args.cpu_seconds > 0:
        def np_of_bytes(t):
            import numpy as np
            t = t.detach().cpu()
            if t.dtype in (torch.float16, torch.bfloat16):
                return t.view(torch.int16).numpy().view(np.uint16)
            return t.numpy()
        hosts = [HostUnit(u, np_of_bytes) for u in pool]
        cpu = cpu_baseline(cfg, hosts, per_elt, args.state, ohp, min_seconds=args.cpu_seconds, blocks=cfg.blocks)
        if args.cpu_all_cores_seconds > 0:
            try:
                host_threads = len(os.sched_getaffinity(0))
            except (AttributeError, OSError):
                host_threads = os.cpu_count() or 1
            if host_threads > 1:
                cpu_all = cpu_baseline(cfg, hosts, per_elt, args.state, ohp, threads=host_threads,
                                       min_seconds=args.cpu_all_cores_seconds, blocks=cfg.blocks)
        del hosts

    ckpt = None
    if args.checkpoint:
        os.makedirs(args.checkpoint, exist_ok=True)
        nbytes = sum(3 * u.S * u.master.element_size() for u in pool)
        torch.cuda.synchronize()
        t_s = time.perf_counter()
        paths = []
        for b, u in enumerate(pool):
            path = ss.shard_path(os.path.join(args.checkpoint, "%s-unit%d" % (cfg.name, b)), 0)
            ss.save_shard(path, cfg.numels, cfg.world, 0, u.master, u.m, u.v, step=args.warmup + args.steps,
                          hp=hp, compute_dtype=u.compute.dtype)
            paths.append(path)
        save_s = time.perf_counter() - t_s
        t_l = time.perf_counter()
        for path, u in zip(paths, pool):
            ss.load_shard(path, u.master, u.m, u.v)
        load_s = time.perf_counter() - t_l
        for path in paths:
            os.remove(path)
        ckpt = {"units": len(pool), "bytes": nbytes, "save_s": round(save_s, 4), "load_s": round(load_s, 4),
                "save_gbps": round(nbytes / save_s / 1e9, 3), "load_gbps": round(nbytes / load_s / 1e9, 3),
                "note": "blocking calls: device-to-host through pinned staging, CRC32C, file write + fsync "
                        "(load: read, CRC32C, host-to-device)"}

    P = pool[0].P
    del per_unit, groups, pool
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    flat = flatten_rate(cfg, ss, torch, N, lib, workloads, args.state)
    unflat = unflatten_rate(cfg, ss, torch, N, lib, workloads, args.state)
    out = {
        "metric": METRIC, "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "config": {"workload": "%s x%d" % (cfg.name, cfg.blocks), "pipeline": args.pipeline,
                   "optimizer": args.optimizer, "state_dtype": args.state,
                   "streams": len(streams),
                   "world": cfg.world, "rank": 0,
                   "shard_numel": S, "unit_numel": P, "blocks_per_step": cfg.blocks,
                   "distinct_blocks": cfg.pool, "grad_dtype": cfg.grad_dt,
                   "fp32_reduce_scatter": cfg.fp32_reduce, "compute_dtype": cfg.compute_dt,
                   "gathers_per_step": G, "bytes_per_shard_element": per_elt,
                   "bytes_per_step": bytes_step},
        "shard_elements_per_s": round(S * cfg.blocks / (ms_step * 1e-3), 1),
        "unit_elements_per_s": round(cfg.world * S * cfg.blocks / (ms_step * 1e-3), 1),
        "wall_s_timed": round(wall, 3),
        "flatten": flat,
        "unflatten": unflat,
        "roofline": roof,
        "cpu_baseline": cpu,
        "cpu_all_cores": cpu_all,
        "checkpoint": ckpt,
    }
    return out




def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures the one-GPU hot path only; --gpus %d is not supported "
              "(run with --gpus 1)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.state != "f32" and args.pipeline in ("separate", "offload"):
        print("--state %s needs --pipeline units or unit" % args.state, file=sys.stderr)
        sys.exit(2)
    if args.optimizer != "adamw" and (args.pipeline != "units" or args.state != "f32"):
        print("--optimizer %s needs --pipeline units and fp32 state" % args.optimizer, file=sys.stderr)
        sys.exit(2)
    import torch
    import sharded_state_amd as ss
    from sharded_state_amd import _native as N
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    lib = N.lib()
    torch.cuda.set_device(0)

    if args.probe == "copy":
        print(json.dumps(dict(probe="copy", **copy_ceiling(torch, N, lib))))
        return

    names = ORDER if args.workload == "all" else [args.workload]
    results = {}
    for name in names:
        t0 = time.perf_counter()
        results[name] = run_workload(args, workloads.CONFIGS[name], torch, ss, N, lib, workloads)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        r = results[name]
        print("bench: %s done in %.1f s: %.1f GB/s (%s)" % (r["config"]["workload"], time.perf_counter() - t0,
                                                          r["value"], r.get("pct_hbm_peak", "-")),
              file=sys.stderr, flush=True)
    head = results[HEADLINE if args.workload == "all" else args.workload]
    out = dict(head)
    if args.pipeline != "offload":
        ceil = copy_ceiling(torch, N, lib)
        ceil["frac_of_peak"] = round(ceil["gbps"] / HBM_PEAK_GBPS, 4)
        ceil["step_frac_of_copy"] = round(head["value"] / ceil["gbps"], 4)
        out["copy_ceiling"] = ceil
    if args.workload == "all":
        keep = ("value", "unit", "ms_per_step", "pct_hbm_peak", "config", "shard_elements_per_s", "roofline",
                "cpu_baseline", "cpu_all_cores", "flatten", "unflatten")
        out["configs"] = {n: {k: r.get(k) for k in keep} for n, r in results.items()}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
