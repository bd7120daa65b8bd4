"""Pins for the oracle's AdamW step and for the whole per-rank step.

The pages write the update only as W = W - lr * Adam(G_avg, m, v) ("Data
Parallelism", section "The Basic Protocol"); the reading is the published AdamW
(bias-corrected Adam, weight decay decoupled as p * (1 - lr*wd), eps after the
square root).  It is pinned by:
  * torch.optim.AdamW (an independent library implementation) over many steps
    and at steps t in {1, 10, 1000}, to a few ulps;
  * the t = 1, m = v = 0 closed form p(1 - lr*wd) - lr*g/(|g| + eps);
  * special cases (g = 0; lr = 0; all-zero padding stays +0);
  * exact rational arithmetic with every operation rounded to fp32 (pins "one
    IEEE fp32 operation per step, no FMA, correctly rounded sqrt and divide");
  * FSDP gives the same result as DDP ("Fully Sharded Data Parallel: faster AI
    training with fewer GPUs", end of section "From all-reduce to sharded
    parameters"; "fairseq 中的 FSDP 实战指南", DDP comparison): sharded steps over
    all N ranks, gathered, equal the unsharded step bit for bit, for every N.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from exact import f32, round_to, sqrt_rounded


def _hp_tuple(h):
    return dict(lr=h.lr, betas=(h.beta1, h.beta2), eps=h.eps, weight_decay=h.weight_decay)


def _torch_adamw(p0, grads, h, m0=None, v0=None, t0=0):
    p = torch.tensor(p0, dtype=torch.float32, requires_grad=True)
    opt = torch.optim.AdamW([p], foreach=False, fused=False, **_hp_tuple(h))
    if m0 is not None:
        opt.state[p] = {"step": torch.tensor(float(t0)), "exp_avg": torch.tensor(m0),
                        "exp_avg_sq": torch.tensor(v0)}
    for g in grads:
        p.grad = torch.tensor(g, dtype=torch.float32)
        opt.step()
    st = opt.state[p]
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


def test_matches_torch_adamw_over_twenty_steps(orc):
    rng = np.random.default_rng(0)
    n = 20000
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    grads = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(20)]
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t, g in enumerate(grads, start=1):
        orc.adamw(p, m, v, g, orc.hp(step=t))
    tp, tm, tv = _torch_adamw(p0, grads, orc.hp())
    # m is a running sum of signed terms of size ~1e-4 (cancellation), so its
    # tolerance is a few fp32 ulps of the terms per step, in absolute terms
    np.testing.assert_allclose(m, tm, rtol=1e-5, atol=2e-10)
    np.testing.assert_allclose(v, tv, rtol=1e-5, atol=1e-16)
    np.testing.assert_allclose(p, tp, rtol=1e-6, atol=3e-8)


@pytest.mark.parametrize("t", [1, 10, 1000])
def test_matches_torch_adamw_at_step_t(orc, t):
    rng = np.random.default_rng(t)
    n = 20000
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    h = orc.hp(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=t)
    p, m, v = p0.copy(), m0.copy(), v0.copy()
    orc.adamw(p, m, v, g, h)
    tp, tm, tv = _torch_adamw(p0, [g], h, m0, v0, t0=t - 1)
    np.testing.assert_allclose(m, tm, rtol=2e-6, atol=5e-11)   # ulps of the ~1e-4 terms
    np.testing.assert_allclose(v, tv, rtol=2e-6, atol=1e-17)
    np.testing.assert_allclose(p, tp, rtol=1e-6, atol=1e-8)


def test_first_step_closed_form(orc):
    """t = 1, m = v = 0: m_hat = g and sqrt(v_hat) = |g|, so
    p' = p(1 - lr*wd) - lr * g / (|g| + eps)."""
    rng = np.random.default_rng(1)
    n = 5000
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-9, -2, n)).astype(np.float32)
    lr, wd, eps = 1e-3, 0.01, 1e-8
    h = orc.hp(lr=lr, weight_decay=wd, eps=eps)
    pp, m, v = p.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    orc.adamw(pp, m, v, g, h)
    P, G = p.astype(np.float64), g.astype(np.float64)
    lr32, wd32, eps32 = (float(np.float32(x)) for x in (lr, wd, eps))
    want = P * (1 - lr32 * wd32) - lr32 * G / (np.abs(G) + eps32)
    u = 2.0 ** -24
    assert np.all(np.abs(pp - want) <= 8 * u * (np.abs(P) + lr32))
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.999))   # hyper-parameters are fp32
    np.testing.assert_allclose(m, (1 - b1) * G, rtol=4 * u)
    np.testing.assert_allclose(v, (1 - b2) * G * G, rtol=8 * u)


def test_zero_grad_zero_state_is_pure_decay(orc):
    rng = np.random.default_rng(2)
    p = (rng.standard_normal(1000) * 0.02).astype(np.float32)
    z = np.zeros(1000, np.float32)
    pp, m, v = p.copy(), z.copy(), z.copy()
    orc.adamw(pp, m, v, z, orc.hp(step=3))
    decay = np.float32(1.0 - float(np.float32(1e-3)) * float(np.float32(0.01)))
    assert np.array_equal(pp, p * decay)
    assert not np.any(m) and not np.any(v)


def test_zero_lr_leaves_params_bitwise(orc):
    rng = np.random.default_rng(3)
    p = (rng.standard_normal(1000) * 0.02).astype(np.float32)
    pp, m, v = p.copy(), np.zeros(1000, np.float32), np.zeros(1000, np.float32)
    orc.adamw(pp, m, v, (rng.standard_normal(1000) * 1e-3).astype(np.float32), orc.hp(lr=0.0))
    assert pp.tobytes() == p.tobytes()
    assert np.all(m != 0) and np.all(v > 0)


def test_padding_stays_positive_zero(orc):
    z = np.zeros(64, np.float32)
    p, m, v = z.copy(), z.copy(), z.copy()
    for t in (1, 2, 3):
        orc.adamw(p, m, v, z, orc.hp(step=t))
    for a in (p, m, v):
        assert a.view(np.uint32).tolist() == [0] * 64


def test_nan_inf_propagation(orc):
    p = np.array([0.1, 0.1, np.nan, 0.1], np.float32)
    g = np.array([np.nan, np.inf, 1e-3, 0.0], np.float32)
    m = np.zeros(4, np.float32)
    v = np.zeros(4, np.float32)
    orc.adamw(p, m, v, g, orc.hp())
    assert np.isnan(p[0]) and np.isnan(p[1]) and np.isnan(p[2]) and np.isfinite(p[3])


def _adamw_exact(p, m, v, g, scalars):
    """The update with every fp32 operation done exactly and rounded once."""
    decay, b1, omb1, b2, omb2, step, bc2s, eps = (f32(x) for x in scalars)
    R = lambda x: round_to(x, "f32")  # noqa: E731
    p, m, v, g = f32(p), f32(m), f32(v), f32(g)
    p1 = R(p * decay)
    m1 = R(R(b1 * m) + R(omb1 * g))
    v1 = R(R(b2 * v) + R(omb2 * R(g * g)))
    den = R(R(sqrt_rounded(v1, "f32") / bc2s) + eps)
    p2 = R(p1 - R(step * R(m1 / den)))
    return p2, m1, v1


def test_eight_elements_against_exact_rationals(orc):
    rng = np.random.default_rng(8)
    h = orc.hp(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=7)
    p = (rng.standard_normal(8) * 0.02).astype(np.float32)
    m = (rng.standard_normal(8) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(8) * 1e-7).astype(np.float32)
    g = (rng.standard_normal(8) * 1e-3).astype(np.float32)
    g[0] = 0.0
    g[1] = np.float32(6e-8)                # tiny gradient: v1 subnormal-adjacent
    pp, mm, vv = p.copy(), m.copy(), v.copy()
    orc.adamw(pp, mm, vv, g, h)
    s = orc.adamw_scalars(h)
    # host scalars: decay and bias terms computed in double, rounded once
    assert Fraction(float(s[0])) == round_to(1 - Fraction(float(np.float32(1e-3))) * f32(0.01), "f32")
    for i in range(8):
        want = _adamw_exact(p[i], m[i], v[i], g[i], s)
        assert (f32(pp[i]), f32(mm[i]), f32(vv[i])) == want, i


@pytest.mark.parametrize("grad_dt,fp32,compute_dt", [
    ("f32", True, "f32"), ("f16", True, "f16"), ("bf16", False, "bf16"), ("f16", False, "bf16")])
def test_sharded_step_equals_unsharded_step_for_every_world(orc, grad_dt, fp32, compute_dt):
    """DDP: all-reduce, then AdamW and cast on the full buffer.  FSDP: each rank
    reduce-scatters, steps its own shard and casts it; the gather of the compute
    shards equals DDP's compute copy, and the master/m/v shards concatenate to
    DDP's, bit for bit, whatever N is (the optimizer is pointwise)."""
    rng = np.random.default_rng(9)
    P = 4999
    params = (rng.standard_normal(P) * 0.02).astype(np.float32)
    for world in (1, 2, 3, 8):
        Pp = orc.padded_numel(P, world)
        S = Pp // world
        master = np.zeros(Pp, np.float32)
        master[:P] = params
        grads = []
        for _ in range(world):
            x = np.zeros(Pp, np.float32)
            x[:P] = (rng.standard_normal(P) * 1e-4).astype(np.float32)
            grads.append(x if grad_dt == "f32" else orc.f32_to(x, grad_dt))
        h = orc.hp(step=2)
        # DDP reference
        avg = orc.all_reduce(grads, grad_dt, fp32)
        g32 = avg if avg.dtype == np.float32 else orc.to_f32(avg, grad_dt)
        dp, dm, dv = master.copy(), np.zeros(Pp, np.float32), np.zeros(Pp, np.float32)
        orc.adamw(dp, dm, dv, g32, h)
        ddp_compute = orc.cast(dp, compute_dt)
        # FSDP, every rank
        shards_c, shards_p, shards_m, shards_v = [], [], [], []
        for r in range(world):
            ps = master[r * S:(r + 1) * S].copy()
            ms, vs = np.zeros(S, np.float32), np.zeros(S, np.float32)
            _, c = orc.rank_step(grads, r, ps, ms, vs, h, grad_dt, fp32, compute_dt)
            shards_c.append(c)
            shards_p.append(ps)
            shards_m.append(ms)
            shards_v.append(vs)
        assert orc.gather(shards_c, compute_dt).tobytes() == ddp_compute.tobytes()
        assert np.concatenate(shards_p).tobytes() == dp.tobytes()
        assert np.concatenate(shards_m).tobytes() == dm.tobytes()
        assert np.concatenate(shards_v).tobytes() == dv.tobytes()
        # padding stays +0 in master, m, v
        assert not np.any(dp[P:].view(np.uint32)) and not np.any(dm[P:].view(np.uint32))


def test_elementwise_sample_equals_full_shard(orc):
    """The sampled form used at full sizes (inputs gathered at chosen positions)
    equals the shard computation at those positions."""
    rng = np.random.default_rng(10)
    world, S = 2, 3000
    grads = [orc.f32_to((rng.standard_normal(world * S) * 1e-4).astype(np.float32), "bf16")
             for _ in range(world)]
    master = (rng.standard_normal(world * S) * 0.02).astype(np.float32)
    h = orc.hp()
    r = 1
    ps = master[r * S:(r + 1) * S].copy()
    ms, vs = np.zeros(S, np.float32), np.zeros(S, np.float32)
    _, c = orc.rank_step(grads, r, ps, ms, vs, h, "bf16", False, "bf16")
    idx = np.sort(rng.choice(S, 200, replace=False))
    pos = r * S + idx
    sp = master[pos].copy()
    sm, sv = np.zeros(200, np.float32), np.zeros(200, np.float32)
    _, sc = orc.elementwise_step([g[pos] for g in grads], sp, sm, sv, h, "bf16", False, "bf16")
    assert sp.tobytes() == ps[idx].tobytes() and sc.tobytes() == c[idx].tobytes()


@pytest.mark.parametrize("state_dt", ["bf16", "f16"])
def test_16bit_state_is_the_fp32_update_rounded_once(orc, state_dt):
    """AdamW on 16-bit state = the fp32 AdamW on the widened values, each result
    rounded once to the state format (both pinned above)."""
    rng = np.random.default_rng(12)
    n = 50000
    p16 = orc.f32_to((rng.standard_normal(n) * 0.02).astype(np.float32), state_dt)
    m16 = orc.f32_to((rng.standard_normal(n) * 1e-3).astype(np.float32), state_dt)
    v16 = orc.f32_to(np.abs(rng.standard_normal(n) * 1e-4).astype(np.float32), state_dt)
    g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    h = orc.hp(step=5)
    p, m, v = p16.copy(), m16.copy(), v16.copy()
    orc.adamw16(p, m, v, g, h, state_dt)
    P, M, V = (orc.to_f32(x, state_dt) for x in (p16, m16, v16))
    orc.adamw(P, M, V, g, h)
    assert np.array_equal(p, orc.f32_to(P, state_dt))
    assert np.array_equal(m, orc.f32_to(M, state_dt))
    assert np.array_equal(v, orc.f32_to(V, state_dt))


def test_16bit_state_against_torch_adamw_in_fp32(orc):
    """torch.optim.AdamW in fp32 on the widened bf16 state, rounded to bf16,
    agrees within one bf16 ulp (the fp32 sequences differ by a few fp32 ulps)."""
    rng = np.random.default_rng(13)
    n = 20000
    p16 = orc.f32_to((rng.standard_normal(n) * 0.02).astype(np.float32), "bf16")
    m16 = orc.f32_to((rng.standard_normal(n) * 1e-3).astype(np.float32), "bf16")
    v16 = orc.f32_to(np.abs(rng.standard_normal(n) * 1e-4).astype(np.float32), "bf16")
    g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    h = orc.hp(step=3)
    p, m, v = p16.copy(), m16.copy(), v16.copy()
    orc.adamw16(p, m, v, g, h, "bf16")
    tp, tm, tv = _torch_adamw(orc.to_f32(p16, "bf16"), [g], h, orc.to_f32(m16, "bf16"),
                              orc.to_f32(v16, "bf16"), t0=2)
    for got, ref in ((p, tp), (m, tm), (v, tv)):
        r = orc.f32_to(ref, "bf16").astype(np.int32)
        d = np.abs(np.where(r & 0x8000, -(r & 0x7FFF), r & 0x7FFF)
                   - np.where(got.astype(np.int32) & 0x8000, -(got.astype(np.int32) & 0x7FFF),
                              got.astype(np.int32) & 0x7FFF))
        assert d.max() <= 1
