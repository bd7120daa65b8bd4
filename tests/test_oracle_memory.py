"""Pin for the oracle's per-worker memory accounting: the pages' printed 70B
numbers (tests/golden/memory_closed_forms.txt, each line cites its page and
section), plus the invariant every page agrees on: a sharded class holds 1/N of
the padded unit, so N shards hold the unsharded bytes plus the padding."""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "memory_closed_forms.txt")


def _rows():
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        f = line.split(None, 9)
        yield (f[0], int(f[1]), int(f[2]), int(f[3]), float(f[4]), float(f[5]), float(f[6]), float(f[7]),
               float(f[8]))


@pytest.mark.parametrize("row", list(_rows()), ids=lambda r: r[0])
def test_pages_70b_numbers(orc, row):
    case, sp, sg, so, pb, gb, ob, printed, exact = row
    out = orc.memory_per_worker(70_000_000_000, 8, sp, sg, so, pb, gb, ob)
    total_gb = out.sum() / 1e9
    assert total_gb == pytest.approx(exact, rel=1e-12)
    assert total_gb == pytest.approx(printed, rel=0.015)


def test_pure_16bit_state_is_half_of_the_fp32_optimizer_classes(orc):
    """Dropping the fp32 master and keeping m, v in 16 bits: per shard element
    2 (parameter) + 4 (m, v) bytes against 2 + 12 with fp32 master, m, v."""
    pure = orc.memory_per_worker(855_638_016, 8, 1, 1, 1, 2, 0, 4).sum()
    mixed = orc.memory_per_worker(855_638_016, 8, 1, 1, 1, 2, 0, 12).sum()
    assert pure * 14 == mixed * 6


@pytest.mark.parametrize("numel,world", [(1_000_000, 2), (19_677_440, 2), (7, 3), (1, 8), (855_638_016, 8)])
def test_sharded_classes_scale_by_one_over_n(orc, numel, world):
    full = orc.memory_per_worker(numel, world, 0, 0, 0, 2.0, 4.0, 12.0)
    shard = orc.memory_per_worker(numel, world, 1, 1, 1, 2.0, 4.0, 12.0)
    pad = orc.padded_numel(numel, world) - numel
    assert np.allclose(world * shard, full + pad * np.array([2.0, 4.0, 12.0]), rtol=0, atol=0)
