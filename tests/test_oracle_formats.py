"""Pins for the oracle's number-format converters.

The oracle's fp32 -> fp16 and fp32 -> bf16 converters are its own code (bit
fields and integer round-to-nearest-even).  They are pinned against two
independent library routines: numpy's IEEE binary16 cast and torch's bfloat16
cast, both round-to-nearest-even.  NaN inputs are compared by NaN-ness only.
The compute cast (``oracle.cast``: master shard -> compute copy, "FSDP (Fully
Sharded Data Parallel)", section "Mixed Precision and FSDP") is pinned on the
same walks through its own entry point and dtype routing: binary16 against
numpy, bfloat16 against torch, fp32 as the identity on the bit pattern.

By default a stride-7 walk over all 2^32 fp32 bit patterns is checked (every
residue of the low bits, every exponent, both signs); FSDP_EXHAUSTIVE=1 checks
every pattern.
"""
import os

import numpy as np
import pytest
import torch

STRIDE = 1 if os.environ.get("FSDP_EXHAUSTIVE") == "1" else 7
CHUNK = 1 << 26


def _patterns():
    total = 1 << 32
    start = 0
    while start < total:
        idx = np.arange(start, min(start + CHUNK * STRIDE, total), STRIDE, dtype=np.uint64)
        yield idx.astype(np.uint32)
        start += CHUNK * STRIDE


def _nan16(h, bf16):
    if bf16:
        return ((h & 0x7F80) == 0x7F80) & ((h & 0x7F) != 0)
    return ((h & 0x7C00) == 0x7C00) & ((h & 0x3FF) != 0)


def test_f16_to_f32_exhaustive(orc):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.to_f32(h, "f16")
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_to_f32_exhaustive(orc):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.to_f32(h, "bf16")
    ref = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _check16(got, ref, x, u, bf16, what):
    nan = np.isnan(x)
    assert got.dtype == np.uint16 and got.shape == x.shape, what
    assert np.array_equal(_nan16(got, bf16), nan), what
    bad = np.nonzero(got[~nan] != ref[~nan])[0]
    assert bad.size == 0, "%s: first mismatch at fp32 pattern 0x%08x" % (what, u[~nan][bad[0]])


def test_f32_to_f16_against_numpy(orc):
    for u in _patterns():
        x = u.view(np.float32)
        with np.errstate(over="ignore", invalid="ignore"):
            ref = x.astype(np.float16).view(np.uint16)
        _check16(orc.f32_to(x, "f16"), ref, x, u, False, "f32_to f16")
        _check16(orc.cast(x, "f16"), ref, x, u, False, "cast f16")


def test_f32_to_bf16_against_torch(orc):
    for u in _patterns():
        x = u.view(np.float32)
        ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        _check16(orc.f32_to(x, "bf16"), ref, x, u, True, "f32_to bf16")
        _check16(orc.cast(x, "bf16"), ref, x, u, True, "cast bf16")


def test_cast_f32_is_identity(orc):
    """A compute copy in fp32 (the tiny unit's) is the master itself, bit for
    bit; NaNs stay NaNs."""
    for u in _patterns():
        x = u.view(np.float32)
        got = orc.cast(x, "f32")
        assert got.dtype == np.float32 and got.shape == x.shape
        nan = np.isnan(x)
        assert np.array_equal(np.isnan(got), nan)
        bad = np.nonzero(got.view(np.uint32)[~nan] != u[~nan])[0]
        assert bad.size == 0, "first mismatch at fp32 pattern 0x%08x" % u[~nan][bad[0]]


def test_cast_routes_each_dtype(orc):
    """1 + 2^-8 + 2^-10 separates the three routes: bfloat16 keeps 7 fraction
    bits (rounds up to 1 + 2^-7), binary16 keeps all of it, fp32 is exact."""
    x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -10, -3.0], np.float32)
    assert orc.cast(x, "bf16").tolist() == [0x3F81, 0xC040]
    assert orc.cast(x, "f16").tolist() == [0x3C05, 0xC200]
    assert orc.cast(x, "f32").view(np.uint32).tolist() == [0x3F80A000, 0xC0400000]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_round_trip_of_representable_values(orc, dt):
    """Every finite 16-bit value converts to fp32 and back to itself."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    keep = ~_nan16(h, dt == "bf16")
    back = orc.f32_to(orc.to_f32(h[keep], dt), dt)
    assert np.array_equal(back, h[keep])


def test_f16_boundaries_by_hand(orc):
    """Binary16 facts from its definition: max finite 65504, ties to even at the
    overflow threshold 65520, smallest subnormal 2^-24, half of it ties to 0."""
    cases = {
        65504.0: 0x7BFF, 65519.99: 0x7BFF, 65520.0: 0x7C00, -65520.0: 0xFC00,
        2.0 ** -24: 0x0001, 2.0 ** -25: 0x0000, 1.5 * 2.0 ** -25: 0x0001,
        3 * 2.0 ** -25: 0x0002, 2.0 ** -14: 0x0400, 1.0: 0x3C00, -0.0: 0x8000,
        1.0 + 2.0 ** -11: 0x3C00, 1.0 + 3 * 2.0 ** -11: 0x3C02,
    }
    for x, want in cases.items():
        assert int(orc.f32_to(np.array([x], np.float32), "f16")[0]) == want, x
        assert int(orc.cast(np.array([x], np.float32), "f16")[0]) == want, x
