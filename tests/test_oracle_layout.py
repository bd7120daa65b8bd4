"""Pins for the oracle's layout functions (flatten, pad, offsets, unflatten,
gather).

These are bit copies, so they are pinned against numpy's own concatenation and
splitting, against brute force over every split of tiny units, and against the
round-trip invariant: unflattening a flattened unit gives back every tensor
bit for bit, and the padding is +0.
"""
import itertools

import numpy as np
import pytest

from oracle import NP_STORAGE


def _rand(rng, n, dt):
    if dt == "f32":
        return rng.standard_normal(n).astype(np.float32)
    return rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)


def test_padded_numel_is_smallest_multiple(orc):
    for total in range(0, 40):
        for world in range(1, 10):
            want = next(p for p in itertools.count(total) if p % world == 0)
            assert orc.padded_numel(total, world) == want


def test_offsets_are_prefix_sums(orc):
    rng = np.random.default_rng(0)
    n = rng.integers(0, 1000, size=50)
    assert np.array_equal(orc.offsets(n), np.concatenate([[0], np.cumsum(n)[:-1]]))


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("world", [1, 2, 3, 7, 8])
def test_flatten_matches_numpy_concatenate(orc, dt, world):
    rng = np.random.default_rng(world)
    shapes = [(13, 7), (1,), (999,), (4, 4, 3), (0,), (5,)]
    ts = [_rand(rng, int(np.prod(s)), dt).reshape(s) for s in shapes]
    flat = orc.flatten_pad(ts, world, dt)
    cat = np.concatenate([t.reshape(-1) for t in ts])
    pad = (-cat.size) % world
    want = np.concatenate([cat, np.zeros(pad, dtype=NP_STORAGE[dt])])
    assert flat.dtype == want.dtype and flat.view(np.uint8).tobytes() == want.view(np.uint8).tobytes()
    back = orc.unflatten(flat, shapes, dt)
    for a, b in zip(back, ts):
        assert a.shape == b.shape and a.tobytes() == b.tobytes()


def test_brute_force_every_split_of_tiny_units(orc):
    """Every composition of P <= 9 into tensors, every N <= 8: flatten places
    element i of tensor k at offset(k) + i, pads with +0, and unflatten inverts."""
    for P in range(0, 10):
        base = np.arange(1, P + 1, dtype=np.float32)
        for cuts in range(1 << max(P - 1, 0)):
            sizes, cur = [], 1
            for b in range(P - 1):
                if cuts >> b & 1:
                    sizes.append(cur)
                    cur = 1
                else:
                    cur += 1
            if P:
                sizes.append(cur)
            parts, pos = [], 0
            for s in sizes:
                parts.append(base[pos:pos + s].copy())
                pos += s
            for world in range(1, 9):
                flat = orc.flatten_pad(parts, world, "f32")
                assert flat.size % world == 0 and flat.size - P < world
                assert np.array_equal(flat[:P], base)
                assert flat[P:].view(np.uint32).tolist() == [0] * (flat.size - P)
                back = orc.unflatten(flat, [(s,) for s in sizes], "f32")
                assert all(np.array_equal(a, b) for a, b in zip(back, parts))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gather_is_concatenation_in_rank_order(orc, dt):
    rng = np.random.default_rng(3)
    for world in (1, 2, 3, 8):
        S = 37
        shards = [_rand(rng, S, dt) for _ in range(world)]
        full = orc.gather(shards, dt)
        assert full.tobytes() == np.concatenate(shards).tobytes()
        for q in range(world):
            assert full[q * S:(q + 1) * S].tobytes() == shards[q].tobytes()
