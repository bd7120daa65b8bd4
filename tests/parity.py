"""Shared helpers of the GPU parity tests: run one FSDP unit through the HIP path
(all N simulated ranks) and through the oracle on the same seeded inputs, and
compare to the stated bar:
  * flatten, pad, reduce-scatter, gather and unflatten: bit-exact;
  * AdamW fp32 master, m, v: max relative error <= 1e-6, where the relative
    error is |x - ref| / |ref| and ref == 0 requires x == ref exactly;
  * 16-bit outputs: at most 1 ulp (distance of the ordered integer encodings);
  * NaN matches NaN (NaN-ness only).
"""
import numpy as np
import torch

import oracle
import sharded_state_amd as ss
from workloads import TORCH_DTYPE, moments, param_tensors, rank_grad

REL_TOL = 1e-6
ULP_TOL = 1


def np_of(t):
    """Device or host tensor -> numpy storage array (uint16 for 16-bit)."""
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def dt_name(dtype):
    return {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[dtype]


def assert_bitexact(got, ref, what):
    got, ref = np.asarray(got), np.asarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if got.dtype == np.float32:
        gn, rn = np.isnan(got), np.isnan(ref)
        assert np.array_equal(gn, rn), "%s: NaN positions differ" % what
        got, ref = got[~gn], ref[~rn]
        bad = np.nonzero(got.view(np.uint32) != ref.view(np.uint32))[0]
    else:
        bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, "%s: %d mismatches, first at %d: %r vs %r" % (
        what, bad.size, bad[0], got[bad[0]], ref[bad[0]])


def assert_rel(got, ref, what, tol=REL_TOL):
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float32)
    gn, rn = np.isnan(got), np.isnan(ref)
    assert np.array_equal(gn, rn), "%s: NaN positions differ" % what
    g, r = got[~gn].astype(np.float64), ref[~rn].astype(np.float64)
    zero = r == 0
    assert np.array_equal(g[zero], r[zero]), "%s: nonzero where the oracle has 0" % what
    inf = np.isinf(r)
    assert np.array_equal(g[inf], r[inf]), "%s: infinities differ" % what
    keep = ~zero & ~inf
    if keep.any():
        rel = np.abs(g[keep] - r[keep]) / np.abs(r[keep])
        worst = rel.max()
        assert worst <= tol, "%s: max relative error %.3g > %.1g" % (what, worst, tol)


def _ordered16(h, bf16):
    h = h.astype(np.int32)
    sign = (h & 0x8000) != 0
    mag = h & 0x7FFF
    return np.where(sign, -mag, mag)


def assert_ulp16(got, ref, dt, what, tol=ULP_TOL):
    got, ref = np.asarray(got, np.uint16), np.asarray(ref, np.uint16)
    bf = dt == "bf16"
    nanmask = ((ref & 0x7F80) == 0x7F80) & ((ref & 0x7F) != 0) if bf else \
        ((ref & 0x7C00) == 0x7C00) & ((ref & 0x3FF) != 0)
    gnan = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0) if bf else \
        ((got & 0x7C00) == 0x7C00) & ((got & 0x3FF) != 0)
    assert np.array_equal(nanmask, gnan), "%s: NaN positions differ" % what
    d = np.abs(_ordered16(got[~nanmask], bf) - _ordered16(ref[~nanmask], bf))
    assert d.size == 0 or d.max() <= tol, "%s: %d ulp" % (what, d.max())


def compare_compute(got, ref, dt, what):
    if dt == "f32":
        assert_rel(got, ref, what)
    else:
        assert_ulp16(got, ref, dt, what)


class UnitRun:
    """One unit's inputs (seeded, host copies kept) and the GPU and oracle
    results for every rank."""

    def __init__(self, cfg, block=0, device="cuda", gen_device="cpu"):
        self.cfg = cfg
        self.device = device
        self.numels = cfg.numels
        P, Pp, S = ss.fsdp_layout(self.numels, cfg.world)
        self.P, self.Pp, self.S = P, Pp, S
        self.params = [t.to(device) for t in param_tensors(cfg, block, gen_device)]
        self.grads = [rank_grad(cfg, block, q, Pp, gen_device).to(device) for q in range(cfg.world)]
        m, v = moments(cfg, block, 0, Pp, P, gen_device)
        self.m0, self.v0 = m.to(device), v.to(device)
        self.gdt = dt_name(self.grads[0].dtype)
        self.cdt_torch = TORCH_DTYPE[cfg.compute_dt]

    def hp(self, step=None):
        c = self.cfg
        return ss.AdamWHP(c.lr, c.beta1, c.beta2, c.eps, c.weight_decay, step or c.step)

    def run_gpu(self, step=None):
        c, S = self.cfg, self.S
        flat = ss.fsdp_flatten_pad(self.params, c.world)
        self.flat0 = flat.clone()
        self.master = flat.clone()
        self.m, self.v = self.m0.clone(), self.v0.clone()
        self.compute = [torch.empty(S, dtype=self.cdt_torch, device=self.device) for _ in range(c.world)]
        self.gshard = []
        for r in range(c.world):
            self.gshard.append(ss.fsdp_reduce_scatter_local(self.grads, r, c.fp32_reduce, shard_numel=S))
            sl = slice(r * S, (r + 1) * S)
            ss.fsdp_sharded_adamw(self.master[sl], self.m[sl], self.v[sl], self.grads, r, c.fp32_reduce,
                                  self.hp(step), compute_shard=self.compute[r])
        self.full = ss.fsdp_unshard_gather(self.compute)
        self.views = ss.fsdp_unflatten_views(self.full, self.cfg.shapes)
        self.mat = ss.fsdp_unflatten_views(self.full, self.cfg.shapes, materialize=True)
        torch.cuda.synchronize()

    def run_gpu_step_unit(self, step=None, persistent=False):
        """Every rank again from the same initial state, each through the
        one-launch fsdp_step_unit with the peers' compute shards of run_gpu."""
        c, S = self.cfg, self.S
        self.su_master = self.flat0.clone()
        self.su_m, self.su_v = self.m0.clone(), self.v0.clone()
        self.su_full, self.su_compute = [], []
        for r in range(c.world):
            sl = slice(r * S, (r + 1) * S)
            full = torch.empty(c.world * S, dtype=self.cdt_torch, device=self.device)
            cs = torch.empty(S, dtype=self.cdt_torch, device=self.device) if persistent else None
            peers = [None if q == r else self.compute[q] for q in range(c.world)]
            ss.fsdp_step_unit(self.su_master[sl], self.su_m[sl], self.su_v[sl], self.grads, r,
                              c.fp32_reduce, self.hp(step), peers, full, compute_shard=cs)
            self.su_full.append(full)
            self.su_compute.append(cs)
        torch.cuda.synchronize()

    def compare_step_unit(self):
        c = self.cfg
        for name, got, ref in (("master", self.su_master, self.o_master), ("exp_avg", self.su_m, self.o_m),
                               ("exp_avg_sq", self.su_v, self.o_v)):
            g = np_of(got)
            assert_rel(g, ref, "step_unit " + name)
            assert_bitexact(g, ref, "step_unit %s (bit-exact)" % name)
        full_ref = np_of(self.full)
        for r in range(c.world):
            f = np_of(self.su_full[r])
            assert_bitexact(f, full_ref, "step_unit full buffer, rank %d" % r)
            compare_compute(f, self.o_full, c.compute_dt, "step_unit full vs oracle, rank %d" % r)
            if self.su_compute[r] is not None:
                assert_bitexact(np_of(self.su_compute[r]), np_of(self.compute[r]),
                                "step_unit persistent compute shard, rank %d" % r)

    def run_oracle(self, step=None):
        c, S = self.cfg, self.S
        gd = self.gdt
        params = [np_of(t).reshape(-1) for t in self.params]
        self.o_flat = oracle.flatten_pad(params, c.world, "f32")
        grads = [np_of(g) for g in self.grads]
        self.o_master = self.o_flat.copy()
        self.o_m, self.o_v = np_of(self.m0), np_of(self.v0)
        h = oracle.hp(c.lr, c.beta1, c.beta2, c.eps, c.weight_decay, step or c.step)
        self.o_gshard, self.o_compute = [], []
        for r in range(c.world):
            sl = slice(r * S, (r + 1) * S)
            p, m, v = self.o_master[sl].copy(), self.o_m[sl].copy(), self.o_v[sl].copy()
            gs, comp = oracle.rank_step(grads, r, p, m, v, h, gd, c.fp32_reduce, c.compute_dt)
            self.o_master[sl], self.o_m[sl], self.o_v[sl] = p, m, v
            self.o_gshard.append(gs)
            self.o_compute.append(comp)
        self.o_full = oracle.gather(self.o_compute, c.compute_dt)
        self.o_unflat = oracle.unflatten(self.o_full, self.cfg.shapes, c.compute_dt)

    def compare(self, strict_adamw=True):
        c = self.cfg
        assert_bitexact(np_of(self.flat0), self.o_flat, "flatten")
        for r in range(c.world):
            assert_bitexact(np_of(self.gshard[r]), self.o_gshard[r], "reduce-scatter rank %d" % r)
        for name, got, ref in (("master", self.master, self.o_master), ("exp_avg", self.m, self.o_m),
                               ("exp_avg_sq", self.v, self.o_v)):
            g = np_of(got)
            assert_rel(g, ref, name)
            if strict_adamw:
                assert_bitexact(g, ref, name + " (bit-exact)")
        for r in range(c.world):
            compare_compute(np_of(self.compute[r]), self.o_compute[r], c.compute_dt, "compute rank %d" % r)
        full = np_of(self.full)
        # the gather itself is a bit copy of the GPU's own shards
        assert_bitexact(full, np.concatenate([np_of(x) for x in self.compute]), "gather")
        compare_compute(full, self.o_full, c.compute_dt, "gathered full buffer")
        for k, (v, m, o) in enumerate(zip(self.views, self.mat, self.o_unflat)):
            assert tuple(v.shape) == tuple(o.shape)
            assert_bitexact(np_of(m).reshape(-1), np_of(v).reshape(-1), "unflatten copy %d" % k)
            compare_compute(np_of(v).reshape(-1), o.reshape(-1), c.compute_dt, "view %d" % k)


def host_threads(cap=16):
    """Host threads this process may use (at most `cap`)."""
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def oracle_rank_step_threaded(grads, p, m, v, h, grad_dt, fp32_reduce, compute_dt, threads=None):
    """One rank's step by the oracle on whole shards, over disjoint chunks on
    several host threads (the oracle's C calls run outside the GIL; the step is
    pointwise, so chunking changes no value).  grads[q] holds rank q's gradient
    block of this rank (storage arrays); p, m, v (fp32) are updated in place.
    Returns (averaged gradient shard, compute shard)."""
    from concurrent.futures import ThreadPoolExecutor
    oracle.lib()
    S = p.size
    avg_dt = "f32" if (fp32_reduce or grad_dt == "f32") else grad_dt
    avg = np.empty(S, dtype=oracle.NP_STORAGE[avg_dt])
    comp = np.empty(S, dtype=oracle.NP_STORAGE[compute_dt])
    threads = threads or host_threads()
    parts = max(1, min(S // 4096, 4 * threads)) if S else 0
    bounds = [S * k // parts for k in range(parts + 1)] if parts else [0]

    def work(k):
        lo, hi = bounds[k], bounds[k + 1]
        if hi <= lo:
            return
        a = oracle.grad_average(grads, lo, hi - lo, grad_dt, fp32_reduce)
        avg[lo:hi] = a
        g32 = a if a.dtype == np.float32 else oracle.to_f32(a, grad_dt)
        oracle.adamw(p[lo:hi], m[lo:hi], v[lo:hi], g32, h)
        comp[lo:hi] = oracle.cast(p[lo:hi], compute_dt)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(work, range(parts)))
    return avg, comp


def assert_compute_close(got, ref, dt, what):
    """The compute-copy bar on whole buffers: equal encodings pass at once;
    otherwise only the differing positions are checked (<= 1 ulp, fp32 rel)."""
    got, ref = np.asarray(got), np.asarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if dt == "f32":
        if np.array_equal(got.view(np.uint32), ref.view(np.uint32)):
            return
        diff = np.nonzero(got.view(np.uint32) != ref.view(np.uint32))[0]
        assert_rel(got[diff], ref[diff], what)
        return
    if np.array_equal(got, ref):
        return
    diff = np.nonzero(got != ref)[0]
    assert_ulp16(got[diff], ref[diff], dt, what)


def assert_bits_equal(got, ref, what):
    """Whole-buffer bit equality without float temporaries (NaN payloads included)."""
    got, ref = np.asarray(got), np.asarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    view = np.uint32 if got.dtype.itemsize == 4 else np.uint16
    a, b = got.view(view), ref.view(view)
    if not np.array_equal(a, b):
        bad = np.nonzero(a != b)[0]
        raise AssertionError("%s: %d of %d differ, first at %d: 0x%x vs 0x%x"
                             % (what, bad.size, a.size, bad[0], int(a[bad[0]]), int(b[bad[0]])))


def oracle_chunks(S, fn, threads=None):
    """fn(lo, hi) over disjoint chunks of [0, S) on several host threads (the
    oracle's C calls run outside the GIL; every step here is pointwise, so the
    chunking changes no value)."""
    from concurrent.futures import ThreadPoolExecutor
    oracle.lib()
    threads = threads or host_threads()
    parts = max(1, min(S // 4096, 4 * threads)) if S else 0
    bounds = [S * k // parts for k in range(parts + 1)] if parts else [0]
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda k: fn(bounds[k], bounds[k + 1]), range(parts)))
