"""Pins for the oracle's other pointwise optimizers: SGD (plain, heavy-ball
momentum with dampening, Nesterov), Adamax and Adadelta.

"fairseq 中的 FSDP 实战指南", section "限制与兼容性说明": FSDP supports the
pointwise optimizers (Adam, AdamW, Adadelta, Adamax, SGD, ...) because each
rank can update its own shard alone; the pages give none of the updates, so the
reading is the published algorithms as torch.optim documents them, with weight
decay added to the gradient.  Pinned by:
  * torch.optim (an independent library implementation) run in float64 over
    several steps, the fp32 oracle within a few fp32 ulps of it;
  * closed forms (constant gradient: momentum's geometric series; first steps
    of Adamax and Adadelta from zero state);
  * exact rational arithmetic with every operation rounded to fp32 (operation
    order, single rounding, no FMA);
  * invariants: the first momentum buffer is the gradient itself; Adamax's u is
    a decaying running maximum floored at eps; zero gradient and zero parameter
    stay +0 (padding); a zero weight decay is skipped, not multiplied; the
    sharded step over all N ranks equals the unsharded step bit for bit.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from exact import f32, round_to, sqrt_rounded

U = 2.0 ** -24
R = lambda x: round_to(x, "f32")  # noqa: E731


def _torch_run(kind, p0, grads, o, f64=True):
    dt = torch.float64 if f64 else torch.float32
    p = torch.tensor(p0.astype(np.float64) if f64 else p0, dtype=dt, requires_grad=True)
    hp32 = lambda x: float(np.float32(x))  # noqa: E731  (the oracle's hyper-parameters are fp32)
    if kind == "sgd":
        opt = torch.optim.SGD([p], lr=hp32(o.lr), momentum=hp32(o.momentum), dampening=hp32(o.dampening),
                              weight_decay=hp32(o.weight_decay), nesterov=bool(o.nesterov), foreach=False)
    elif kind == "adamax":
        opt = torch.optim.Adamax([p], lr=hp32(o.lr), betas=(hp32(o.beta1), hp32(o.beta2)), eps=hp32(o.eps),
                                 weight_decay=hp32(o.weight_decay), foreach=False)
    else:
        opt = torch.optim.Adadelta([p], lr=hp32(o.lr), rho=hp32(o.rho), eps=hp32(o.eps),
                                   weight_decay=hp32(o.weight_decay), foreach=False)
    peak = np.abs(p0.astype(np.float64))
    for g in grads:
        p.grad = torch.tensor(g.astype(np.float64) if f64 else g, dtype=dt)
        opt.step()
        peak = np.maximum(peak, np.abs(p.detach().numpy()))
    st = opt.state[p]
    keys = {"sgd": ("momentum_buffer",), "adamax": ("exp_avg", "exp_inf"), "adadelta": ("square_avg", "acc_delta")}
    states = [st[k].detach().numpy() if st.get(k) is not None else None for k in keys[kind]]
    return p.detach().numpy(), states, peak


def _oracle_run(orc, kind, p0, grads, **kw):
    p = p0.copy()
    s1, s2 = np.zeros_like(p0), np.zeros_like(p0)
    for t, g in enumerate(grads, start=1):
        orc.opt_step(kind, p, s1, s2, g, orc.opt(kind, step=t, **kw))
    return p, s1, s2


CASES = [
    ("sgd", dict()),
    ("sgd", dict(momentum=0.9)),
    ("sgd", dict(momentum=0.9, dampening=0.1, weight_decay=0.01)),
    ("sgd", dict(momentum=0.8, nesterov=True, weight_decay=1e-4, lr=1e-2)),
    ("adamax", dict()),
    ("adamax", dict(weight_decay=0.01, beta2=0.99)),
    ("adadelta", dict()),
    ("adadelta", dict(weight_decay=0.01, rho=0.95, lr=0.5)),
]


@pytest.mark.parametrize("kind,kw", CASES)
def test_matches_torch_optim_in_float64(orc, kind, kw):
    rng = np.random.default_rng(len(str(kw)) + len(kind))
    n, steps = 20000, 6
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    grads = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(steps)]
    p, s1, s2 = _oracle_run(orc, kind, p0, grads, **kw)
    tp, ts, peak = _torch_run(kind, p0, grads, orc.opt(kind, **kw))
    # parameters: one rounding of p per step, at most U|p| with |p| below its
    # largest value along the way, plus a few ulps of the update
    upd = np.abs(tp - p0.astype(np.float64))
    tol = steps * 2 * U * peak + 16 * U * upd
    assert np.all(np.abs(p - tp) <= tol), kind
    if kind == "sgd" and kw.get("momentum"):
        b = ts[0]
        assert np.all(np.abs(s1 - b) <= 8 * U * steps * np.abs(grads).max(0) * 10), "momentum buffer"
    elif kind == "adamax":
        m, u = ts
        assert np.all(np.abs(s1 - m) <= 8 * U * steps * np.abs(grads).max(0)), "exp_avg"
        assert np.all(np.abs(s2 - u) <= 2 * steps * U * np.abs(u)), "exp_inf"   # a rounding per decay
    elif kind == "adadelta":
        v, acc = ts
        assert np.all(np.abs(s1 - v) <= 8 * U * steps * np.abs(np.square(grads)).max(0)), "square_avg"
        assert np.all(np.abs(s2 - acc) <= 64 * U * np.abs(acc) + 1e-30), "acc_delta"
    # the tolerance is far below one step's update, so a dropped or mis-signed
    # term (weight decay, momentum, bias correction) cannot hide in it
    assert np.median(tol) < np.median(upd) / steps / 10


def test_sgd_constant_gradient_geometric_series(orc):
    """Constant gradient g, no weight decay or dampening: b_t = g (1 - mu^t) / (1 - mu)
    and p_t = p_0 - lr * sum_k b_k; Nesterov uses g + mu * b_t instead of b_t."""
    n, T, mu, lr = 512, 12, 0.9, 1e-2
    rng = np.random.default_rng(3)
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    for nesterov in (False, True):
        p, b, _ = _oracle_run(orc, "sgd", p0, [g] * T, momentum=mu, lr=lr, nesterov=nesterov)
        mu32, lr32, G = float(np.float32(mu)), float(np.float32(lr)), g.astype(np.float64)
        bt = [G * (1 - mu32 ** k) / (1 - mu32) for k in range(1, T + 1)]
        steps = [G + mu32 * x for x in bt] if nesterov else bt
        want_p = p0.astype(np.float64) - lr32 * np.sum(steps, axis=0)
        np.testing.assert_allclose(b, bt[-1], rtol=64 * U * T)
        assert np.all(np.abs(p - want_p) <= 16 * U * T * (np.abs(want_p) + lr32 * np.abs(np.sum(steps, 0))))


def test_sgd_first_buffer_is_the_gradient_bitwise(orc):
    """At t = 1 the buffer is the (weight-decayed) gradient itself, whatever the dampening."""
    rng = np.random.default_rng(4)
    p0 = (rng.standard_normal(1000) * 0.02).astype(np.float32)
    g = (rng.standard_normal(1000) * 1e-3).astype(np.float32)
    p, b, _ = _oracle_run(orc, "sgd", p0, [g], momentum=0.9, dampening=0.5)
    assert b.tobytes() == g.tobytes()
    assert p.tobytes() == (p0 - np.float32(1e-3) * g).tobytes()


def test_adamax_first_step_closed_form_and_running_max(orc):
    rng = np.random.default_rng(5)
    n = 4000
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-7, -2, n)).astype(np.float32)
    p, m, u = _oracle_run(orc, "adamax", p0, [g])
    eps, lr = float(np.float32(1e-8)), float(np.float32(2e-3))
    G = g.astype(np.float64)
    # m1 = (1-b1) g, u1 = |g| + eps, p1 = p - lr/(1-b1) * m1/u1 = p - lr g/(|g|+eps)
    np.testing.assert_allclose(u, np.abs(G) + eps, rtol=2 * U)
    want = p0 - lr * G / (np.abs(G) + eps)
    assert np.all(np.abs(p - want) <= 8 * U * (np.abs(p0) + lr))
    # zero gradients afterwards: u decays by beta2 per step and is floored at eps
    z = np.zeros(n, np.float32)
    uu = u.copy()
    pp, mm = p.copy(), m.copy()
    for t in range(2, 40):
        orc.adamax(pp, mm, uu, z, orc.opt("adamax", step=t))
    b2 = float(np.float32(0.999))
    want_u = np.maximum((np.abs(G) + eps) * b2 ** 38, eps)
    np.testing.assert_allclose(uu, want_u, rtol=64 * U)


def test_adadelta_first_step_closed_form(orc):
    rng = np.random.default_rng(6)
    n = 4000
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-6, -1, n)).astype(np.float32)
    p, v, acc = _oracle_run(orc, "adadelta", p0, [g])
    rho, eps = float(np.float32(0.9)), float(np.float32(1e-6))
    G = g.astype(np.float64)
    v1 = (1 - rho) * G * G
    delta = np.sqrt(eps) / np.sqrt(v1 + eps) * G
    np.testing.assert_allclose(v, v1, rtol=4 * U)
    np.testing.assert_allclose(acc, (1 - rho) * delta * delta, rtol=16 * U)
    assert np.all(np.abs(p - (p0 - delta)) <= 8 * U * (np.abs(p0) + np.abs(delta)))


def _exact(kind, p, s1, s2, g, o):
    """The update with every fp32 operation done exactly and rounded once."""
    p, s1, s2, g = f32(p), f32(s1), f32(s2), f32(g)
    wd, lr = f32(o.weight_decay), f32(o.lr)
    d = R(g + R(wd * p)) if wd != 0 else g
    if kind == "sgd":
        mu, omd = f32(o.momentum), R(1 - f32(o.dampening))
        if mu != 0:
            b = d if o.step == 1 else R(R(mu * s1) + R(omd * d))
            s1 = b
            d = R(d + R(mu * b)) if o.nesterov else b
        return R(p - R(lr * d)), s1, s2
    if kind == "adamax":
        b1, b2, eps = f32(o.beta1), f32(o.beta2), f32(o.eps)
        clr = f32(np.float32(float(lr) / (1.0 - float(b1) ** o.step)))       # host: double, rounded once
        m1 = R(R(b1 * s1) + R(R(1 - b1) * d))
        u1 = max(R(b2 * s2), R(abs(d) + eps))
        return R(p - R(clr * R(m1 / u1))), m1, u1
    rho, eps = f32(o.rho), f32(o.eps)
    omr = R(1 - rho)
    v1 = R(R(rho * s1) + R(omr * R(d * d)))
    delta = R(R(sqrt_rounded(R(s2 + eps), "f32") / sqrt_rounded(R(v1 + eps), "f32")) * d)
    a1 = R(R(rho * s2) + R(omr * R(delta * delta)))
    return R(p - R(lr * delta)), v1, a1


@pytest.mark.parametrize("kind,kw", CASES)
@pytest.mark.parametrize("step", [1, 5])
def test_elements_against_exact_rationals(orc, kind, kw, step):
    n = 64
    rng = np.random.default_rng(step * 7 + len(kw))
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    s1 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    s2 = np.abs(rng.standard_normal(n) * 1e-3).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    g[0] = 0.0
    g[1] = np.float32(3e-9)
    if kind == "adadelta":
        s1 = np.abs(s1 * 1e-3)
        s2 = np.abs(s2 * 1e-3)
    o = orc.opt(kind, step=step, **kw)
    pp, a, b = p.copy(), s1.copy(), s2.copy()
    orc.opt_step(kind, pp, a, b, g, o)
    for i in range(n):
        want = _exact(kind, p[i], s1[i], s2[i], g[i], o)
        got = (f32(pp[i]), f32(a[i]), f32(b[i]))
        if kind == "sgd" and not kw.get("momentum"):
            got, want = got[0], want[0]
        assert got == want, (kind, kw, step, i)


@pytest.mark.parametrize("kind", ["sgd", "adamax", "adadelta"])
def test_padding_stays_positive_zero(orc, kind):
    z = np.zeros(64, np.float32)
    p, s1, s2 = z.copy(), z.copy(), z.copy()
    kw = dict(momentum=0.9, weight_decay=0.01) if kind == "sgd" else dict(weight_decay=0.01)
    for t in (1, 2, 3):
        orc.opt_step(kind, p, s1, s2, z, orc.opt(kind, step=t, **kw))
    assert p.view(np.uint32).tolist() == [0] * 64
    if kind == "adamax":                      # u floors at eps; m stays +0
        assert s1.view(np.uint32).tolist() == [0] * 64 and np.all(s2 == np.float32(1e-8))
    else:
        assert s1.view(np.uint32).tolist() == [0] * 64


def test_zero_weight_decay_is_skipped_not_multiplied(orc):
    p = np.array([np.inf, -np.inf, 0.5], np.float32)
    g = np.array([1.0, 1.0, 1.0], np.float32)
    a = p.copy()
    orc.sgd(a, None, g, orc.opt("sgd", lr=0.1))
    assert a[0] == np.inf and a[1] == -np.inf and a[2] == np.float32(0.5) - np.float32(0.1)
    b = p.copy()
    orc.sgd(b, None, g, orc.opt("sgd", lr=0.1, weight_decay=0.01))
    assert np.isnan(b[0]) and np.isnan(b[1])        # g + wd * inf = inf; inf - inf = NaN


def test_adamax_max_propagates_nan(orc):
    p = np.array([0.1, 0.1, 0.1], np.float32)
    m = np.zeros(3, np.float32)
    u = np.array([np.nan, 0.0, 1.0], np.float32)
    g = np.array([1e-3, np.nan, 1e-3], np.float32)
    orc.adamax(p, m, u, g, orc.opt("adamax"))
    assert np.isnan(u[0]) and np.isnan(u[1]) and u[2] == np.float32(0.999)
    assert np.isnan(p[0]) and np.isnan(p[1]) and np.isfinite(p[2])


@pytest.mark.parametrize("kind,kw", [("sgd", dict(momentum=0.9, nesterov=True)), ("adamax", dict()),
                                     ("adadelta", dict(weight_decay=0.01))])
def test_sharded_step_equals_unsharded_step(orc, kind, kw):
    rng = np.random.default_rng(11)
    P = 3001
    for world, grad_dt, fp32 in ((2, "f16", True), (3, "bf16", False), (8, "f32", True)):
        Pp = orc.padded_numel(P, world)
        S = Pp // world
        master = np.zeros(Pp, np.float32)
        master[:P] = (rng.standard_normal(P) * 0.02).astype(np.float32)
        grads = []
        for _ in range(world):
            x = np.zeros(Pp, np.float32)
            x[:P] = (rng.standard_normal(P) * 1e-3).astype(np.float32)
            grads.append(x if grad_dt == "f32" else orc.f32_to(x, grad_dt))
        o = orc.opt(kind, step=2, **kw)
        avg = orc.all_reduce(grads, grad_dt, fp32)
        g32 = avg if avg.dtype == np.float32 else orc.to_f32(avg, grad_dt)
        dp, d1, d2 = master.copy(), np.full(Pp, 1e-4, np.float32), np.full(Pp, 1e-6, np.float32)
        s1_0, s2_0 = d1.copy(), d2.copy()
        orc.opt_step(kind, dp, d1, d2, g32, o)
        for r in range(world):
            sl = slice(r * S, (r + 1) * S)
            ps, a, b = master[sl].copy(), s1_0[sl].copy(), s2_0[sl].copy()
            _, c = orc.rank_step_opt(kind, grads, r, ps, a, b, o, grad_dt, fp32, "bf16")
            assert ps.tobytes() == dp[sl].tobytes() and a.tobytes() == d1[sl].tobytes()
            assert b.tobytes() == d2[sl].tobytes()
            assert c.tobytes() == orc.cast(dp[sl], "bf16").tobytes()
