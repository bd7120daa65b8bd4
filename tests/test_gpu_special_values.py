"""Special values through the fused unit step for every optimizer, on the GPU
against the oracle: NaN, +-Inf, subnormals, signed zeros and values that
overflow binary16 in the parameter, the gradients and the optimizer state;
fp16 and bf16 compute copies.  fp32 outputs must match bit for bit (NaN by
NaN-ness), 16-bit outputs bit for bit away from NaN and NaN-ness at NaN."""
import numpy as np
import pytest
import torch

import oracle
import sharded_state_amd as ss
from parity import assert_bitexact, assert_ulp16, np_of

pytestmark = pytest.mark.gpu

H = ss.OptimHP
OPTS = {
    "adamw": None,
    "sgd": H.sgd(lr=1e-2, weight_decay=1e-4),
    "sgd-wd0": H.sgd(lr=1e-2),
    "sgd-momentum": H.sgd(lr=1e-2, momentum=0.9, dampening=0.1, weight_decay=1e-4),
    "sgd-nesterov": H.sgd(lr=1e-2, momentum=0.9, nesterov=True),
    "adamax": H.adamax(weight_decay=0.01),
    "adadelta": H.adadelta(weight_decay=0.01),
}
SPECIAL = np.array([np.nan, np.inf, -np.inf, 1e-40, -1e-40, 0.0, -0.0, 65504.0, 65520.0, 70000.0, -70000.0,
                    3e38, -3e38, 5.9e-8, 3e-8, 1e-45, 1.0, -1.0], dtype=np.float32)


def _orc(name, hp, step):
    if name == "adamw":
        return "adamw", oracle.hp(step=step)
    if hp.kind == 1:
        return "sgd", oracle.opt("sgd", step=step, lr=hp.lr, weight_decay=hp.weight_decay, momentum=hp.momentum,
                                 dampening=hp.dampening, nesterov=bool(hp.nesterov))
    if hp.kind == 2:
        return "adamax", oracle.opt("adamax", step=step, lr=hp.lr, weight_decay=hp.weight_decay, beta1=hp.beta1,
                                    beta2=hp.beta2, eps=hp.eps)
    return "adadelta", oracle.opt("adadelta", step=step, lr=hp.lr, weight_decay=hp.weight_decay, rho=hp.rho,
                                  eps=hp.eps)


@pytest.mark.parametrize("cdt", ["f16", "bf16"])
@pytest.mark.parametrize("name", list(OPTS))
def test_special_values_every_optimizer(name, cdt):
    world, S = 2, 1003                                 # ragged: the vector body and the scalar tail
    rng = np.random.default_rng(len(name))
    n = world * S

    def with_specials(x, shift):
        x = x.copy()
        for k, val in enumerate(SPECIAL):
            x[(k * 37 + shift) % n] = val
            x[(k * 53 + shift + 900) % n] = val       # also in the other rank's block and the tail
        return x

    p = with_specials((rng.standard_normal(n) * 0.02).astype(np.float32), 0)
    grads = [with_specials((rng.standard_normal(n) * 1e-3).astype(np.float32), 11 + q) for q in range(world)]
    m = with_specials(np.abs(rng.standard_normal(n) * 1e-4).astype(np.float32), 5)
    v = with_specials(np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32), 7)
    ctd = {"f16": torch.float16, "bf16": torch.bfloat16}[cdt]
    hp = OPTS[name]
    gd = [torch.from_numpy(g).cuda() for g in grads]
    for step in (1, 2):
        for r in range(world):
            sl = slice(r * S, (r + 1) * S)
            tp, tm, tv = (torch.from_numpy(x[sl].copy()).cuda() for x in (p, m, v))
            cs = torch.empty(S, dtype=ctd, device="cuda")
            unit = dict(master=tp, exp_avg=tm, exp_avg_sq=tv, rank_grads=gd, compute_shard=cs)
            ss.fsdp_step_units([unit], r, True, ss.AdamWHP(step=step) if hp is None else hp.at_step(step))
            torch.cuda.synchronize()
            kind, o = _orc(name, hp, step)
            op, om, ov = p[sl].copy(), m[sl].copy(), v[sl].copy()
            _, oc = oracle.rank_step_opt(kind, grads, r, op, om, ov, o, "f32", True, cdt)
            what = "%s %s step %d rank %d" % (name, cdt, step, r)
            assert_bitexact(np_of(tp), op, "param, " + what)
            n_states = 2 if hp is None else hp.n_states
            if n_states >= 1:
                assert_bitexact(np_of(tm), om, "state 1, " + what)
            if n_states >= 2:
                assert_bitexact(np_of(tv), ov, "state 2, " + what)
            got = np_of(cs)
            assert_ulp16(got, oc, cdt, "compute, " + what, tol=0)


@pytest.mark.parametrize("sdt", ["bf16", "f16"])
def test_special_values_16bit_state(sdt):
    """The pure 16-bit state step (parameter, m, v stored in bf16 / fp16) with
    special values in every input."""
    world, S = 2, 1003
    rng = np.random.default_rng(3)
    n = world * S
    torch_dt = {"f16": torch.float16, "bf16": torch.bfloat16}[sdt]

    def with_specials(x, shift):
        x = x.copy()
        for k, val in enumerate(SPECIAL):
            x[(k * 41 + shift) % n] = val
        return x

    p = oracle.f32_to(with_specials((rng.standard_normal(n) * 0.02).astype(np.float32), 0), sdt)
    m = oracle.f32_to(with_specials(np.abs(rng.standard_normal(n) * 1e-4).astype(np.float32), 5), sdt)
    v = oracle.f32_to(with_specials(np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32), 9), sdt)
    grads = [with_specials((rng.standard_normal(n) * 1e-3).astype(np.float32), 13 + q) for q in range(world)]
    gd = [torch.from_numpy(g).cuda() for g in grads]
    h = oracle.hp(step=2)
    for r in range(world):
        sl = slice(r * S, (r + 1) * S)
        tp, tm, tv = (torch.from_numpy(x[sl].copy().view(np.int16)).view(torch_dt).cuda() for x in (p, m, v))
        ss.fsdp_step_units([dict(master=tp, exp_avg=tm, exp_avg_sq=tv, rank_grads=gd)], r, True, ss.AdamWHP(step=2))
        torch.cuda.synchronize()
        op, om, ov = p[sl].copy(), m[sl].copy(), v[sl].copy()
        oracle.rank_step16(grads, r, op, om, ov, h, "f32", True, sdt)
        for nm, got, ref in (("param", tp, op), ("exp_avg", tm, om), ("exp_avg_sq", tv, ov)):
            assert_ulp16(np_of(got), ref, sdt, "%s %s rank %d" % (nm, sdt, r), tol=0)


@pytest.mark.parametrize("world", [1, 2, 8, 3])
def test_bf16_reduce_scatter_keeps_nan_payloads(world):
    """bf16 gradients reduced in bf16 (no --fp32-reduce-scatter): signalling and
    quiet NaNs with payloads, of either sign, each alone at its position across
    the ranks, come out of the reduce-scatter as the oracle's quiet NaN with the
    same sign and payload, bit for bit; so do infinities, overflow to infinity
    and the numbers around them.  With one rank no add runs: the signalling NaN
    is quieted by the division by N alone.  Where two ranks' NaNs meet or +Inf meets -Inf
    only NaN-ness is compared (the pages fix no payload there).  Covers the
    vector body and the scalar tail of the reduce-scatter kernel."""
    S = 1003
    print("case bf16 NaN payloads, N=%d" % world, flush=True)
    rng = np.random.default_rng(world)
    n = world * S
    base = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(world)]
    bits = [oracle.f32_to(b, "bf16").copy() for b in base]       # the bf16 encodings
    rank = world - 1
    lo = rank * S
    singles = [0x7F81, 0x7FC5, 0xFF82, 0xFFC3, 0x7FA0, 0xFFFF, 0x7F80, 0xFF80]   # NaNs with payloads, +-Inf
    exact_pos = []
    for k, val in enumerate(singles):
        body = [lo + 5 + 61 * k]
        tail = [lo + S - 1 - k] if k < 3 else []                     # the last 3 elements: the scalar tail
        for pos in body + tail:
            q = (k + pos) % world
            bits[q][pos] = val
            exact_pos.append(pos)
    big = oracle.f32_to(np.array([3.3e38], np.float32), "bf16")[0]
    for q in range(world):                                          # overflow to +Inf in the sum
        bits[q][lo + 700] = big
    exact_pos.append(lo + 700)
    nan_only = []
    if world >= 2:
        bits[0][lo + 800], bits[1][lo + 800] = 0x7F80, 0xFF80       # +Inf + -Inf
        bits[0][lo + 801], bits[1][lo + 801] = 0x7F81, 0xFFC7       # two NaNs meet
        nan_only = [lo + 800, lo + 801]
    grads = [torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).cuda() for b in bits]
    out = ss.fsdp_reduce_scatter_local(grads, rank, False)
    torch.cuda.synchronize()
    got = np_of(out)
    ref = oracle.reduce_scatter(bits, rank, "bf16", False)
    keep = np.ones(S, bool)
    keep[[p - lo for p in nan_only]] = False
    bad = np.nonzero((got != ref) & keep)[0]
    assert bad.size == 0, "bits differ at %s: %s vs %s" % (bad[:8], got[bad[:8]], ref[bad[:8]])
    for p in nan_only:
        isnan = lambda h: (int(h) & 0x7FFF) > 0x7F80
        assert isnan(got[p - lo]) and isnan(ref[p - lo]), (p, hex(got[p - lo]), hex(ref[p - lo]))
    for p in exact_pos:
        assert got[p - lo] == ref[p - lo]


def test_bf16_compute_copy_of_every_fp32_encoding():
    """The bf16 cast of the step, on all 2^32 fp32 encodings of the parameter.
    With lr = 0, zero weight decay, zero gradient and zero moments, the update
    leaves the parameter as it is (p * 1 - 0 * 0; a NaN comes out quiet with its
    payload), so the compute copy is the cast of the parameter itself: it must
    equal the oracle's cast bit for bit everywhere -- ties, subnormals, both
    zeros, infinities and every NaN payload -- and the master must come back as
    the (quieted) input.  Runs the fp32-state unit kernel in 16 launches of 2^28
    elements (the vector path; the tail path is covered by the other tests)."""
    from parity import assert_bits_equal, oracle_chunks
    n = 1 << 28
    dev = "cuda"
    m = torch.zeros(n, device=dev)
    v = torch.zeros(n, device=dev)
    g = torch.zeros(n, device=dev)
    comp = torch.empty(n, dtype=torch.bfloat16, device=dev)
    hp = ss.AdamWHP(lr=0.0, weight_decay=0.0, step=1)
    low = torch.arange(n, dtype=torch.int32, device=dev)
    for c in range(16):
        print("chunk", c, flush=True)
        hi = (c << 28) - (1 << 32) if c >= 8 else c << 28
        master = (low | hi).view(torch.float32)
        ss.fsdp_sharded_adamw(master, m, v, [g], 0, True, hp, compute_shard=comp)
        torch.cuda.synchronize()
        u = (np.arange(n, dtype=np.uint32) | np.uint32(c << 28))
        nan = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)
        quiet = u | (nan.astype(np.uint32) << 22)
        want = np.empty(n, np.uint16)

        def cast(lo, hi_):
            want[lo:hi_] = oracle.cast(quiet[lo:hi_].view(np.float32), "bf16")

        oracle_chunks(n, cast)
        assert_bits_equal(np_of(comp), want, "bf16 cast, encodings 0x%08x.." % (c << 28))
        assert_bits_equal(np_of(master).view(np.uint32), quiet, "master, encodings 0x%08x.." % (c << 28))
        assert not m.any() and not v.any()
