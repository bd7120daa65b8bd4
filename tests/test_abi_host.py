"""The C ABI on the host (no GPU needed): the library loads, exports every
symbol the header declares, and its host-only paths work -- layout sizes, the
view table, and argument validation, which runs before anything touches the
device (fake, never-dereferenced pointers are enough to reach every check)."""
import ctypes
import os
import re

import numpy as np
import pytest

import sharded_state_amd as ss
from sharded_state_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = []
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", f)).read()
            names += re.findall(r"FSDP_API\s+[\w\s\*]+?\b(fsdp_\w+)\s*\(", txt)
    return names


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 8, names
    L = N.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.fsdp_abi_version() == N.ABI_VERSION


def test_layout_matches_oracle(orc):
    rng = np.random.default_rng(0)
    for _ in range(50):
        k = int(rng.integers(1, 12))
        numels = [int(x) for x in rng.integers(0, 5000, size=k)]
        world = int(rng.integers(1, 9))
        P, Pp, S = ss.fsdp_layout(numels, world)
        assert P == sum(numels) and Pp == orc.padded_numel(P, world) and S * world == Pp
        table = ss.view_table(numels, Pp)
        assert [o for o, _ in table] == list(orc.offsets(numels)) and [n for _, n in table] == numels


FAKE = 1 << 40   # device-looking addresses, never dereferenced: validation fails first


def _adamw(master, m, v, grads, world, rank, gdt=N.F16, cdt=N.F16, S=1000, step=1, out=FAKE + (1 << 32)):
    hp = N.AdamWHP(step=step)
    return N.lib().fsdp_sharded_adamw(ctypes.c_void_p(master), ctypes.c_void_p(m), ctypes.c_void_p(v),
                                      N.ptr_array(grads), world, rank, gdt, 1, ctypes.c_void_p(out),
                                      cdt, S, ctypes.byref(hp), None)


def test_validation_errors_before_any_launch():
    L = N.lib()
    g = [FAKE + (1 << 36), FAKE + (2 << 36)]
    a, b, c = FAKE, FAKE + (1 << 30), FAKE + (2 << 30)
    assert _adamw(a, b, c, g, 0, 0) == N.E_INVAL
    assert _adamw(a, b, c, g, 2, 2) == N.E_INVAL
    assert _adamw(a, b, c, g, 2, -1) == N.E_INVAL
    assert _adamw(a, b, c, g, 2, 0, gdt=7) == N.E_DTYPE
    assert _adamw(a, b, c, g, 2, 0, cdt=9) == N.E_DTYPE
    assert _adamw(a, b, c, g, 2, 0, step=0) == N.E_INVAL
    assert _adamw(a, a + 100, c, g, 2, 0) == N.E_ALIAS          # master overlaps exp_avg
    assert _adamw(a, b, c, [a, g[1]], 2, 0) == N.E_ALIAS        # grad block overlaps master
    assert _adamw(a, b, c, g, 2, 0, out=c + 3996) == N.E_ALIAS  # compute overlaps exp_avg_sq
    assert _adamw(0, b, c, g, 2, 0) == N.E_INVAL
    assert _adamw(a, b, c, [g[0], 0], 2, 0) == N.E_INVAL
    assert _adamw(a, b, c, g * 65, 130, 0) == N.E_INVAL          # world above the maximum
    msg = L.fsdp_last_error().decode()
    assert "world" in msg
    # reduce-scatter: output overlapping an input block
    rc = L.fsdp_reduce_scatter_local(N.ptr_array(g), 2, 1, 1000, N.F16, 0,
                                     ctypes.c_void_p(g[0] + 2000), None)
    assert rc == N.E_ALIAS
    # gather: a shard overlapping the output outside its own slot
    full = FAKE
    rc = L.fsdp_unshard_gather(N.ptr_array([full + 2000, FAKE + (1 << 33)]), 2, 1000, N.F16,
                               ctypes.c_void_p(full), None)
    assert rc == N.E_ALIAS
    # flatten: capacity too small, source overlapping the flat buffer
    rc = L.fsdp_flatten_pad(N.ptr_array([FAKE + (1 << 33)]), N.i64_array([10]), 1, N.F32, 4,
                            ctypes.c_void_p(FAKE), 11, None, None)
    assert rc == N.E_SIZE
    rc = L.fsdp_flatten_pad(N.ptr_array([FAKE + 8]), N.i64_array([10]), 1, N.F32, 4,
                            ctypes.c_void_p(FAKE), 12, None, None)
    assert rc == N.E_ALIAS
    # unflatten: more elements than the buffer
    views = (N.View * 2)()
    rc = L.fsdp_unflatten_views(N.i64_array([5, 6]), 2, 10, views, None, N.F32, None, None)
    assert rc == N.E_SIZE


def test_empty_shard_is_a_no_op_without_device_work():
    """shard_numel == 0 returns OK after validation, before any HIP call."""
    assert _adamw(0, 0, 0, [0, 0], 2, 1, S=0, out=0) == N.OK
    L = N.lib()
    assert L.fsdp_reduce_scatter_local(N.ptr_array([0, 0]), 2, 0, 0, N.BF16, 0, None, None) == N.OK
    assert L.fsdp_unshard_gather(N.ptr_array([0]), 1, 0, N.F16, None, None) == N.OK


def test_python_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        ss.fsdp_unshard_gather([torch.zeros(4)])


def _step_unit(peers, full, world=2, rank=0, S=1000, cs=None):
    hp = N.AdamWHP()
    a, b, c = FAKE, FAKE + (1 << 30), FAKE + (2 << 30)
    g = [FAKE + ((3 + q) << 30) for q in range(world)]
    return N.lib().fsdp_step_unit(ctypes.c_void_p(a), ctypes.c_void_p(b), ctypes.c_void_p(c),
                                  N.ptr_array(g), world, rank, N.BF16, 0, N.ptr_array(peers),
                                  ctypes.c_void_p(full), N.BF16, S, ctypes.c_void_p(cs), ctypes.byref(hp),
                                  None)


def test_step_unit_validation():
    full = FAKE + (20 << 30)
    peer = FAKE + (21 << 30)
    assert _step_unit([0, full + 2], full) == N.E_ALIAS             # peer inside the full buffer
    assert _step_unit([0, peer], full, cs=full + 100) == N.E_ALIAS  # extra copy inside full
    assert _step_unit([0, 0], full) == N.E_INVAL                     # missing peer shard
    assert _step_unit([0, peer], 0) == N.E_INVAL                     # missing full buffer
    assert _step_unit([0, peer], full, rank=2) == N.E_INVAL
    assert _step_unit([0, peer], FAKE + 8) == N.E_ALIAS              # full overlaps master


def test_step_units_validation():
    L = N.lib()
    hp = N.AdamWHP()
    g = N.ptr_array([FAKE + (30 << 30), FAKE + (31 << 30)])
    peers = N.ptr_array([0, FAKE + (32 << 30)])

    def unit(base, full):
        return N.Unit(base, base + (1 << 28), base + (2 << 28), g, peers, full, None, 1000)

    a = unit(FAKE, FAKE + (40 << 30))
    b = unit(FAKE + (1 << 30), FAKE + (41 << 30))
    table = (N.Unit * 2)(a, b)
    # distinct units would be launched; here only the error paths are exercised
    dup = (N.Unit * 2)(a, a)
    assert L.fsdp_step_units(dup, 2, 2, 0, N.BF16, 0, N.F32, N.BF16, ctypes.byref(hp), None) == N.E_ALIAS
    mixed = (N.Unit * 2)(a, unit(FAKE + (2 << 30), 0))
    assert L.fsdp_step_units(mixed, 2, 2, 0, N.BF16, 0, N.F32, N.BF16, ctypes.byref(hp), None) == N.E_INVAL
    cross = (N.Unit * 2)(a, unit(FAKE + (3 << 30), FAKE + (1 << 28)))   # b's full overlaps a's exp_avg
    assert L.fsdp_step_units(cross, 2, 2, 0, N.BF16, 0, N.F32, N.BF16, ctypes.byref(hp), None) == N.E_ALIAS
    assert L.fsdp_step_units(table, -1, 2, 0, N.BF16, 0, N.F32, N.BF16, ctypes.byref(hp), None) == N.E_INVAL
    assert L.fsdp_step_units(table, 2, 2, 0, N.BF16, 0, N.F32, 5, ctypes.byref(hp), None) == N.E_DTYPE
    assert L.fsdp_step_units(table, 0, 2, 0, N.BF16, 0, N.F32, N.BF16, ctypes.byref(hp), None) == N.OK
    # 16-bit state: the parameter is the compute copy
    assert L.fsdp_step_units(table, 2, 2, 0, N.BF16, 0, N.BF16, N.F16, ctypes.byref(hp), None) == N.E_DTYPE
    with_cs = (N.Unit * 1)(N.Unit(FAKE, FAKE + (1 << 28), FAKE + (2 << 28), g, peers, FAKE + (40 << 30),
                                  FAKE + (50 << 30), 1000))
    assert L.fsdp_step_units(with_cs, 1, 2, 0, N.BF16, 0, N.BF16, N.BF16, ctypes.byref(hp), None) == N.E_INVAL


def test_step_units_optim_validation():
    """The optimizer entry point checks hyper-parameters and the state buffers
    its optimizer keeps before anything is launched."""
    L = N.lib()
    g = N.ptr_array([FAKE + (30 << 30), FAKE + (31 << 30)])
    peers = N.ptr_array([0, FAKE + (32 << 30)])
    full = FAKE + (40 << 30)

    def call(hp, m=FAKE + (1 << 28), v=FAKE + (2 << 28), state=N.F32, compute=N.BF16, master=FAKE):
        t = (N.Unit * 1)(N.Unit(master, m, v, g, peers, full, None, 1000))
        return L.fsdp_step_units_optim(t, 1, 2, 0, N.BF16, 0, state, compute, ctypes.byref(hp), None)

    H = N.OptimHP
    assert L.fsdp_step_units_optim(None, 0, 2, 0, N.BF16, 0, N.F32, N.BF16, None, None) == N.E_INVAL
    bad = H.sgd()
    bad.kind = 9
    assert call(bad) == N.E_INVAL                                       # unknown optimizer
    assert call(H.sgd(lr=-1.0)) == N.E_INVAL
    assert call(H.sgd(weight_decay=-0.1)) == N.E_INVAL
    assert call(H.sgd(step=0)) == N.E_INVAL
    assert call(H.sgd(momentum=-0.5)) == N.E_INVAL
    assert call(H.sgd(nesterov=True)) == N.E_INVAL                      # Nesterov needs momentum
    assert call(H.sgd(momentum=0.9, dampening=0.1, nesterov=True)) == N.E_INVAL   # ... and no dampening
    assert call(H.adamax(betas=(1.0, 0.999))) == N.E_INVAL
    assert call(H.adamax(eps=-1e-8)) == N.E_INVAL
    assert call(H.adadelta(rho=1.5)) == N.E_INVAL
    assert call(H.adamw(betas=(0.9, 1.0))) == N.E_INVAL
    # 16-bit state is AdamW's only
    for hp in (H.sgd(momentum=0.9), H.adamax(), H.adadelta()):
        assert call(hp, state=N.BF16, compute=N.BF16) == N.E_DTYPE
        assert "AdamW only" in L.fsdp_last_error().decode()
    # the state buffers the optimizer keeps must be given
    assert call(H.sgd(momentum=0.9), m=0) == N.E_INVAL
    assert call(H.adamax(), v=0) == N.E_INVAL
    assert call(H.adadelta(), m=0) == N.E_INVAL
    assert call(H.adamw(), v=0) == N.E_INVAL
    # ... and overlaps are checked among those only: an unused exp_avg_sq may
    # point anywhere (here: into the full buffer) and is never touched, while a
    # used one may not
    assert call(H.adamax(), v=full + 8) == N.E_ALIAS
    assert call(H.sgd(momentum=0.9), m=full + 8) == N.E_ALIAS
    assert call(H.sgd(momentum=0.9), v=full + 8, master=0) == N.E_INVAL   # (stops at master, no launch)
    assert H.sgd().n_states == 0 and H.sgd(momentum=0.9).n_states == 1 and H.adadelta().n_states == 2


def test_unit_gather_split_launch_plan():
    """The launch-plan query: the peers' copies get a launch of their own only
    for an optimizer that keeps state and >= 2^24 shard elements, with fp32 or
    16-bit state alike."""
    import torch
    f32, bf16 = torch.float32, torch.bfloat16
    assert ss.unit_gather_split(f32, 2, 1 << 24)
    assert ss.unit_gather_split(f32, 1, 1 << 30)
    assert not ss.unit_gather_split(f32, 2, (1 << 24) - 1)
    assert not ss.unit_gather_split(f32, 0, 1 << 30)
    assert ss.unit_gather_split(bf16, 2, 1 << 30)
    assert ss.unit_gather_split(torch.float16, 2, 1 << 24)
    assert not ss.unit_gather_split(bf16, 2, (1 << 24) - 1)
    for bad in ((f32, 3, 10), (f32, -1, 10), (f32, 2, -1)):
        with pytest.raises(ss.FsdpError):
            ss.unit_gather_split(*bad)
    lib = ss.lib()
    assert lib.fsdp_unit_gather_split(9, 2, 10) == -2          # FSDP_E_DTYPE


def test_units_in_launch_packing():
    """Packing of a unit-step call: at most 40 / 24 / 16 units (N <= 2 / 4 / 8,
    one unit otherwise) and at most 2^26 shard elements per launch; a larger
    unit is stepped in 2^26-element slices."""
    cap = 1 << 26
    assert ss.units_in_launch(2, []) == (0, 0)
    assert ss.units_in_launch(2, [100] * 50) == (40, 4000)
    assert ss.units_in_launch(1, [100] * 50) == (40, 4000)
    assert ss.units_in_launch(4, [100] * 50) == (24, 2400)
    assert ss.units_in_launch(8, [100] * 50) == (16, 1600)
    assert ss.units_in_launch(3, [100] * 50) == (1, 100)
    assert ss.units_in_launch(2, [9_838_720] * 36) == (6, 6 * 9_838_720)     # GPT-2 Large block shards
    assert ss.units_in_launch(8, [106_954_752] * 2) == (1, cap)             # 70B block shard: slices
    assert ss.units_in_launch(2, [778_804_000]) == (1, cap)                 # GPT-2 XL model shard
    assert ss.units_in_launch(2, [cap, 1]) == (1, cap)                      # exactly at the cap: alone
    assert ss.units_in_launch(2, [cap - 10, 10, 1]) == (2, cap)
    assert ss.units_in_launch(2, [5, cap + 1]) == (1, 5)                    # a larger unit is not packed
    for bad in ((0, [1]), (129, [1]), (2, [-1])):
        with pytest.raises(ss.FsdpError):
            ss.units_in_launch(*bad)


@pytest.mark.parametrize("field,value", [("lr", -1e-3), ("weight_decay", -0.01), ("eps", -1e-8),
                                         ("lr", float("nan")), ("eps", float("nan")),
                                         ("weight_decay", float("nan"))])
def test_every_adamw_entry_point_checks_the_same_hyper_parameters(field, value):
    """lr, weight_decay and eps below 0 (or NaN) are FSDP_E_INVAL at every AdamW
    entry point, as fsdp_step_units_optim already refused them: a negative eps
    could make sqrt(v)/bc2 + eps vanish and turn the update into inf/NaN."""
    L = N.lib()
    hp = N.AdamWHP()
    setattr(hp, field, value)
    hpr = ctypes.byref(hp)
    a, b, c = FAKE, FAKE + (1 << 30), FAKE + (2 << 30)
    g = N.ptr_array([FAKE + (3 << 30), FAKE + (4 << 30)])
    peers = N.ptr_array([0, FAKE + (5 << 30)])
    full = ctypes.c_void_p(FAKE + (6 << 30))
    vp = ctypes.c_void_p
    table = (N.Unit * 1)(N.Unit(a, b, c, g, peers, FAKE + (6 << 30), None, 1000))
    host = [np.zeros(16, np.float32) for _ in range(5)]
    hptr = [vp(x.ctypes.data) for x in host]
    ou = (N.OffloadUnit * 1)(N.OffloadUnit(hptr[0].value, hptr[1].value, hptr[2].value, g, FAKE + (7 << 30),
                                           hptr[3].value, hptr[4].value, FAKE + (8 << 30), 16))
    o = N.OptimHP.adamw()
    setattr(o, field, value)
    calls = {
        "fsdp_sharded_adamw": lambda: L.fsdp_sharded_adamw(vp(a), vp(b), vp(c), g, 2, 0, N.BF16, 0, vp(FAKE + (9 << 30)),
                                                           N.BF16, 1000, hpr, None),
        "fsdp_step_unit": lambda: L.fsdp_step_unit(vp(a), vp(b), vp(c), g, 2, 0, N.BF16, 0, peers, full, N.BF16, 1000,
                                                   None, hpr, None),
        "fsdp_step_units": lambda: L.fsdp_step_units(table, 1, 2, 0, N.BF16, 0, N.F32, N.BF16, hpr, None),
        "fsdp_step_units_optim": lambda: L.fsdp_step_units_optim(table, 1, 2, 0, N.BF16, 0, N.F32, N.BF16,
                                                                 ctypes.byref(o), None),
        "fsdp_host_adamw": lambda: L.fsdp_host_adamw(hptr[0], hptr[1], hptr[2], hptr[3], N.F32, hptr[4], N.F32, 16,
                                                     hpr, 1),
        "fsdp_offload_step": lambda: L.fsdp_offload_step(hptr[0], hptr[1], hptr[2], g, 2, 0, N.BF16, 0,
                                                         vp(FAKE + (7 << 30)), hptr[3], hptr[4], vp(FAKE + (8 << 30)),
                                                         N.BF16, 16, 0, hpr, 1, None, None),
        "fsdp_offload_step_units": lambda: L.fsdp_offload_step_units(ou, 1, 2, 0, N.BF16, 0, N.BF16, 0, hpr, 1, None,
                                                                     None),
    }
    for name, call in calls.items():
        assert call() == N.E_INVAL, name
        assert ">= 0" in L.fsdp_last_error().decode(), name


def test_noalloc_offload_checks_the_scratch_limit_before_any_device_work():
    """The no-allocation offload step refuses a chunk larger than its
    FSDP_OFFLOAD_SCRATCH_BYTES scratch (FSDP_E_SIZE) and a unit that brings its
    own device gradient shard (FSDP_E_INVAL), before touching the device."""
    L = N.lib()
    hp = N.AdamWHP()
    g = N.ptr_array([FAKE + (3 << 30), FAKE + (4 << 30)])
    host = [FAKE + (k << 34) for k in range(1, 6)]

    def call(chunk, fp32_reduce=1, grad_dev=None):
        u = (N.OffloadUnit * 1)(N.OffloadUnit(host[0], host[1], host[2], g, grad_dev, host[3], host[4],
                                              FAKE + (8 << 30), 1000))
        return L.fsdp_offload_step_units_noalloc(u, 1, 2, 0, N.F16, fp32_reduce, N.F16, chunk, ctypes.byref(hp), 1,
                                                 None, None)

    limit = N.OFFLOAD_SCRATCH_BYTES
    assert call(limit // 4 + 8) == N.E_SIZE                  # fp32 average: 4 bytes per element
    assert "scratch" in L.fsdp_last_error().decode()
    assert call(limit // 4 + 1) == N.E_SIZE                  # rounded up to a multiple of 8 first
    assert call(limit // 2 + 8, fp32_reduce=0) == N.E_SIZE   # 16-bit average: 2 bytes per element
    assert call(0, grad_dev=FAKE + (9 << 30)) == N.E_INVAL
    assert "grad_shard_dev must be NULL" in L.fsdp_last_error().decode()


def test_element_counts_whose_byte_offsets_would_wrap_are_refused():
    """A shard times the world, or any buffer, above INT64_MAX / 16 elements is
    refused with FSDP_E_SIZE before any byte offset is formed (fake pointers)."""
    L = N.lib()
    cap = (2 ** 63 - 1) // 16
    g = [FAKE + (1 << 36), FAKE + (2 << 36)]
    a, b, c = FAKE, FAKE + (1 << 30), FAKE + (2 << 30)
    assert _adamw(a, b, c, g, 2, 0, S=cap // 2 + 1) == N.E_SIZE
    assert "too large" in L.fsdp_last_error().decode()
    assert _adamw(a, b, c, g, 2, 0, S=cap // 2, step=0) == N.E_INVAL   # at the bound: the next check speaks
    rc = L.fsdp_reduce_scatter_local(N.ptr_array(g), 2, 1, cap // 2 + 1, N.F16, 0, ctypes.c_void_p(FAKE), None)
    assert rc == N.E_SIZE
    rc = L.fsdp_unshard_gather(N.ptr_array(g), 2, cap // 2 + 1, N.F16, ctypes.c_void_p(FAKE), None)
    assert rc == N.E_SIZE
    views = (N.View * 1)()
    rc = L.fsdp_unflatten_views(N.i64_array([5]), 1, cap + 1, views, None, N.F32, None, None)
    assert rc == N.E_SIZE
    rc = L.fsdp_flatten_pad(N.ptr_array([FAKE, FAKE]), N.i64_array([cap, 1]), 2, N.F32, 1,
                            ctypes.c_void_p(FAKE), 2 ** 62, None, None)
    assert rc == N.E_SIZE
    hp = N.AdamWHP()
    host = [FAKE + (k << 34) for k in range(1, 6)]
    u = (N.OffloadUnit * 1)(N.OffloadUnit(host[0], host[1], host[2], N.ptr_array(g), FAKE + (9 << 30), host[3],
                                          host[4], FAKE + (8 << 30), cap // 2 + 1))
    rc = L.fsdp_offload_step_units(u, 1, 2, 0, N.F16, 1, N.F16, 0, ctypes.byref(hp), 1, None, None)
    assert rc == N.E_SIZE
