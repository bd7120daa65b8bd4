"""The host AdamW kernel of the CPU-offload path (fsdp_host_adamw), on the CPU.

The offloaded step keeps the fp32 master and the AdamW moments in host memory
and updates them there; its result must be the one the device kernels and the
oracle give, bit for bit: every grad dtype, every compute dtype (and none),
one and several worker threads, lengths with ragged 8-lane tails, unaligned
buffers, and special values (subnormals, signed zeros, binary16 overflow).
"""
import ctypes

import numpy as np
import pytest
import torch

import sharded_state_amd as ss
from sharded_state_amd import _native as N
from parity import assert_bitexact, dt_name, np_of

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _inputs(n, seed, grad_dt, scale=1e-3):
    g = torch.Generator().manual_seed(seed)
    p = torch.randn(n, generator=g) * 0.02
    m = torch.randn(n, generator=g).abs() * 1e-4
    v = torch.randn(n, generator=g).abs() * 1e-4
    grad = (torch.randn(n, generator=g) * scale).to(DT[grad_dt])
    return p, m, v, grad


def _oracle(orc, p, m, v, grad, h, compute_dt):
    P, M, V = np_of(p), np_of(m), np_of(v)
    gn = np_of(grad)
    g32 = gn if grad.dtype == torch.float32 else orc.to_f32(gn, dt_name(grad.dtype))
    orc.adamw(P, M, V, g32, h)
    C = orc.cast(P, compute_dt) if compute_dt else None
    return P, M, V, C


def _check(orc, p, m, v, grad, step, compute_dt, threads):
    h = orc.hp(step=step)
    P, M, V, C = _oracle(orc, p, m, v, grad, h, compute_dt)
    c = torch.empty(p.numel(), dtype=DT[compute_dt]) if compute_dt else None
    ss.fsdp_host_adamw(p, m, v, grad, ss.AdamWHP(step=step), compute=c, n_threads=threads)
    assert_bitexact(np_of(p), P, "master")
    assert_bitexact(np_of(m), M, "exp_avg")
    assert_bitexact(np_of(v), V, "exp_avg_sq")
    if compute_dt:
        assert_bitexact(np_of(c), C, "compute (%s)" % compute_dt)


@pytest.mark.parametrize("grad_dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("compute_dt", ["f32", "f16", "bf16", None])
@pytest.mark.parametrize("threads", [1, 5])
def test_host_adamw_matches_oracle(orc, grad_dt, compute_dt, threads):
    n = 300_007                                     # ragged tail of every range split
    _check(orc, *_inputs(n, 11, grad_dt), step=7, compute_dt=compute_dt, threads=threads)


@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 8191, 8192, 16385])
def test_host_adamw_lengths(orc, n):
    _check(orc, *_inputs(n, n, "bf16"), step=1, compute_dt="bf16", threads=3)


def test_host_adamw_unaligned_views(orc):
    """Buffers starting at odd element offsets (loads and stores unaligned)."""
    n = 100_003
    base = [t for t in _inputs(n + 3, 5, "f16")]
    p, m, v, g = base[0][1:n + 1], base[1][2:n + 2], base[2][3:n + 3], base[3][1:n + 1]
    _check(orc, p, m, v, g, step=2, compute_dt="f16", threads=4)


def test_host_adamw_special_values(orc):
    """Subnormal and zero gradients, subnormal and overflowing binary16 compute
    values, negative zero: the vector body and the scalar tail (n % 8 != 0) both
    see every case."""
    vals = np.array([0.0, -0.0, 1e-40, -1e-40, 1e-45, 3e-39, 1e-8, 65504.0, 65519.0, 65520.0, 70000.0,
                     -70000.0, 6e-8, 5.96e-8, 2.98e-8, 1e-5, 6.1e-5, -6.1e-5, 3e38, -3e38, 1.0, -1.0],
                    dtype=np.float32)
    n = vals.size * 8 + 5
    p = torch.from_numpy(np.resize(vals, n).copy())
    g = torch.from_numpy(np.resize(vals[::-1], n).copy())
    m = torch.from_numpy(np.resize(vals * 1e-3, n).copy()).abs()
    with np.errstate(over="ignore"):
        v = torch.from_numpy(np.resize(vals * vals, n).astype(np.float32))      # includes +inf
    for cdt in ("f16", "bf16"):
        _check(orc, p.clone(), m.clone(), v.clone(), g.clone(), step=3, compute_dt=cdt, threads=2)
        for lo in range(0, n, 7):                                             # scalar path only
            sl = slice(lo, min(n, lo + 7))
            _check(orc, p[sl].clone(), m[sl].clone(), v[sl].clone(), g[sl].clone(), step=3, compute_dt=cdt,
                   threads=1)
    _check(orc, p.clone(), m.clone(), v.clone(), g.to(torch.bfloat16), step=1, compute_dt="f16", threads=1)


@pytest.mark.parametrize("compute_dt", ["f16", "bf16"])
def test_host_cast_of_every_exponent(orc, compute_dt):
    """With lr = 0 the master passes through unchanged, so the compute copy is
    the rounding of arbitrary fp32 values (random encodings over every exponent,
    NaN excluded): vector body over the whole array, scalar path over runs of 7."""
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 32, size=60_000, dtype=np.uint64).astype(np.uint32)
    bits = bits[(bits & 0x7F800000) != 0x7F800000]
    # plus ties and near-ties at the binary16 / bfloat16 rounding points
    near = rng.integers(0, 1 << 20, size=4000, dtype=np.uint64).astype(np.uint32)
    ties = np.concatenate([(near << 13) | 0x1000, (near << 16) | 0x8000, (near << 13) | 0x0FFF])
    ties = ties[(ties & 0x7F800000) != 0x7F800000]
    p0 = torch.from_numpy(np.concatenate([bits, ties]).view(np.float32).copy())
    n = p0.numel()
    g = torch.full((n,), 1e-3)
    h = orc.hp(lr=0.0, weight_decay=0.0)
    c = torch.empty(n, dtype=DT[compute_dt])
    ss.fsdp_host_adamw(p0.clone(), torch.zeros(n), torch.zeros(n), g, ss.AdamWHP(lr=0.0, weight_decay=0.0),
                       compute=c, n_threads=4)
    P = np_of(p0)
    orc.adamw(P, np.zeros(n, np.float32), np.zeros(n, np.float32), np_of(g), h)
    assert_bitexact(np_of(p0), P, "master unchanged")
    want = orc.cast(P, compute_dt)
    assert_bitexact(np_of(c), want, "vector cast")
    c7 = torch.empty(n, dtype=DT[compute_dt])
    for lo in range(0, 7 * 400, 7):
        sl = slice(lo, lo + 7)
        ss.fsdp_host_adamw(p0[sl].clone(), torch.zeros(7), torch.zeros(7), g[sl], ss.AdamWHP(lr=0.0, weight_decay=0.0),
                           compute=c7[sl], n_threads=1)
    assert_bitexact(np_of(c7)[:2800], want[:2800], "scalar cast")
    tail = slice(n - 2800, n)                                                   # the ties, scalar path
    for lo in range(tail.start, n, 7):
        sl = slice(lo, min(n, lo + 7))
        ss.fsdp_host_adamw(p0[sl].clone(), torch.zeros(sl.stop - lo), torch.zeros(sl.stop - lo), g[sl],
                           ss.AdamWHP(lr=0.0, weight_decay=0.0), compute=c7[sl], n_threads=1)
    assert_bitexact(np_of(c7)[tail], want[tail], "scalar cast of ties")


def test_host_adamw_many_steps_stay_identical(orc):
    n = 40_000
    p, m, v, _ = _inputs(n, 3, "f32")
    P, M, V = np_of(p), np_of(m), np_of(v)
    for t in range(1, 6):
        grad = _inputs(n, 100 + t, "bf16")[3]
        h = orc.hp(step=t)
        gn = orc.to_f32(np_of(grad), "bf16")
        orc.adamw(P, M, V, gn, h)
        ss.fsdp_host_adamw(p, m, v, grad, ss.AdamWHP(step=t), n_threads=3)
    assert_bitexact(np_of(p), P, "master after 5 steps")
    assert_bitexact(np_of(v), V, "exp_avg_sq after 5 steps")


def test_host_adamw_validation():
    L = N.lib()
    n = 64
    a = [np.zeros(n, np.float32) for _ in range(4)]
    ptr = [ctypes.c_void_p(x.ctypes.data) for x in a]
    hp = N.AdamWHP()

    def call(p=ptr[0], m=ptr[1], v=ptr[2], g=ptr[3], gdt=N.F32, c=None, cdt=N.F32, nn=n, h=hp, th=2):
        return L.fsdp_host_adamw(p, m, v, g, gdt, c, cdt, nn, ctypes.byref(h) if h is not None else None, th)

    assert call() == N.OK
    assert call(nn=-1) == N.E_INVAL
    assert call(gdt=7) == N.E_DTYPE
    assert call(cdt=5, c=ptr[3]) == N.E_DTYPE
    assert call(h=None) == N.E_INVAL
    assert call(h=N.AdamWHP(step=0)) == N.E_INVAL
    assert call(h=N.AdamWHP(beta1=1.0)) == N.E_INVAL
    assert call(p=None) == N.E_INVAL
    assert call(m=ptr[0]) == N.E_ALIAS
    assert call(c=ctypes.c_void_p(a[2].ctypes.data + 8)) == N.E_ALIAS   # compute inside exp_avg_sq
    assert "overlap" in L.fsdp_last_error().decode()
    assert call(nn=0, p=None) == N.OK                                    # empty: nothing is touched
    with pytest.raises(ValueError):
        ss.fsdp_host_adamw(torch.zeros(4), torch.zeros(4), torch.zeros(3), torch.zeros(4), ss.AdamWHP())
    with pytest.raises(TypeError):
        ss.fsdp_host_adamw(torch.zeros(4, dtype=torch.float16), torch.zeros(4), torch.zeros(4), torch.zeros(4),
                           ss.AdamWHP())


def test_offload_step_units_validation_before_any_device_work():
    """Argument checks of the offloaded batch step run before anything touches
    the device: fake, never-dereferenced device addresses reach every check."""
    L = N.lib()
    S, world = 4096, 2
    FAKE = 1 << 40
    host = [np.zeros(S, np.float32) for _ in range(10)]

    def unit(k, grads=None, gdev=None, cdev=None, master=None, S=S):
        h = host[5 * k:5 * k + 5] if k < 2 else host[:5]
        gp = N.ptr_array(grads if grads is not None else [FAKE + (k * 8 + q) * (1 << 30) for q in range(world)])
        u = N.OffloadUnit(master if master is not None else h[0].ctypes.data, h[1].ctypes.data, h[2].ctypes.data,
                          gp, gdev if gdev is not None else FAKE + (100 + 2 * k) * (1 << 30), h[3].ctypes.data,
                          h[4].ctypes.data, cdev if cdev is not None else FAKE + (101 + 2 * k) * (1 << 30), S)
        return u, gp

    def call(units, n=None, world=world, rank=0, gdt=N.F32, cdt=N.F32, hp=N.AdamWHP()):
        table = (N.OffloadUnit * max(1, len(units)))(*[u for u, _ in units])
        return L.fsdp_offload_step_units(table if units else None, len(units) if n is None else n, world, rank, gdt,
                                         1, cdt, 0, ctypes.byref(hp), 2, None, None)

    assert call([]) == N.OK
    assert call([], n=-1) == N.E_INVAL
    assert call([unit(0)], world=0) == N.E_INVAL
    assert call([unit(0)], rank=2) == N.E_INVAL
    assert call([unit(0)], gdt=9) == N.E_DTYPE
    assert call([unit(0)], hp=N.AdamWHP(step=0)) == N.E_INVAL
    assert call([unit(0, master=0)]) == N.E_INVAL
    assert call([unit(0, grads=[FAKE, 0])]) == N.E_INVAL
    assert call([unit(0, S=0)]) == N.OK                               # empty unit: nothing to do
    # the same host state twice in one batch
    assert call([unit(0), unit(2)]) == N.E_ALIAS
    # a device output on top of another unit's output, or of a gradient block it reads
    u1 = unit(1, gdev=FAKE + 100 * (1 << 30) + 64)
    assert call([unit(0), u1]) == N.E_ALIAS
    u1 = unit(1, cdev=FAKE + (0 * 8 + 1) * (1 << 30))                   # rank 1's grad block 0 of unit 0
    assert call([unit(0), u1]) == N.E_ALIAS
    assert "overlap" in L.fsdp_last_error().decode()
