"""bench.py's host logic (no GPU): the byte accounting against the closed forms
of the algorithmic bytes per shard element, the counter-summary key, the buffer
rotation of the flatten and unflatten rates, and the refusal of more than one
GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import CONFIGS  # noqa: E402


def _canonical(cfg):
    """Bytes per shard element when every buffer is touched once and each gather
    reads and writes all N shards: N*g + 12 (read master, m, v) + 12 (write) +
    c (own compute shard) + G * 2N*c."""
    g = 4 if cfg.grad_dt == "f32" else 2
    c = 4 if cfg.compute_dt == "f32" else 2
    return cfg.world * g + 24 + c + cfg.gathers * 2 * cfg.world * c


@pytest.mark.parametrize("name,expected", [("tiny", 52), ("gpt2-large-block", 38), ("gpt2-xl-model", 38),
                                           ("gpt3-13b-block", 106), ("llama70b-block", 74)])
def test_canonical_bytes_per_element(name, expected):
    cfg = CONFIGS[name]
    assert _canonical(cfg) == expected
    # the three-launch pipeline moves exactly the canonical bytes
    assert bench.sizes(cfg, "separate")[1] == expected


@pytest.mark.parametrize("name", ["tiny", "gpt2-large-block", "gpt2-xl-model", "gpt3-13b-block", "llama70b-block"])
@pytest.mark.parametrize("split", [False, True])
def test_unit_step_bytes_skip_only_the_own_shard_copy(name, split):
    """The unit step writes its own compute shard once, straight into its slot
    of the full buffer, and the first gather never reads it back: with one
    gather that is 2c bytes fewer than the canonical count (the reduced count
    N*g + 24 + (2N-1)*c); with two gathers the step also writes the persistent
    own copy the second gather reads, c fewer.  Nothing else differs, and the
    timed kernel carries the peers' copies unless they run in their own launch."""
    cfg = CONFIGS[name]
    c = 4 if cfg.compute_dt == "f32" else 2
    kernel, step = bench.sizes(cfg, "unit", "f32", 2, split)
    assert step == _canonical(cfg) - (2 * c if cfg.gathers == 1 else c)
    if cfg.gathers == 1:
        assert step == cfg.world * (4 if cfg.grad_dt == "f32" else 2) + 24 + (2 * cfg.world - 1) * c
    peers = 2 * (cfg.world - 1) * c
    others = (cfg.gathers - 1) * 2 * cfg.world * c
    assert kernel == step - others - (peers if split else 0)


def test_state_buffers_change_only_the_state_bytes():
    cfg = CONFIGS["gpt2-large-block"]
    k2, s2 = bench.sizes(cfg, "unit", "f32", 2, True)
    k1, s1 = bench.sizes(cfg, "unit", "f32", 1, True)
    k0, s0 = bench.sizes(cfg, "unit", "f32", 0, False)
    assert (k2 - k1, s2 - s1) == (8, 8)
    assert s1 - s0 == 8
    assert k0 == s0                      # SGD keeps the copies in its trip: the kernel is the whole step


def test_sixteen_bit_state_bytes():
    cfg = CONFIGS["llama70b-block"]      # N = 8, bf16 grads and compute
    kernel, step = bench.sizes(cfg, "unit", "bf16")
    assert kernel == step == 8 * 2 + 12 + 2 + 2 * 7 * 2
    # were the launch plan to split the peers' copies out, the step launch would not carry them
    ks, ss_ = bench.sizes(cfg, "unit", "bf16", 2, True)
    assert (ks, ss_) == (8 * 2 + 12 + 2, step)
    g2 = CONFIGS["gpt3-13b-block"]       # two gathers: the second one's bytes are in the step only
    k2, s2 = bench.sizes(g2, "unit", "f16")
    assert k2 == 8 * 2 + 12 + 2 + 2 * 7 * 2 and s2 == k2 + 2 * 8 * 2


def test_kernel_code_ignores_comments_only():
    a = "int x; // one\n/* two\n three */ int y;\n\n"
    b = "int x;\n int y; // other words\n"
    assert bench.kernel_code(a) == "int x;\n int y;"
    assert bench.kernel_code(a) == bench.kernel_code(b)
    assert bench.kernel_code("int x;") != bench.kernel_code("int z;")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one-GPU" in r.stderr and not r.stdout


def test_cpu_baseline_whole_units_and_extrapolation():
    """The oracle baseline runs on the host alone over whole units (every unit
    of the pool once per pass), on one pinned core or on several threads over
    disjoint chunks, and counts the GPU line's bytes per shard element; with
    fewer distinct units than slots per step it says it extrapolates."""
    import types
    import torch
    cfg = CONFIGS["gpt2-large-block"]           # N = 2, fp16 grads reduced in fp32, fp16 compute
    S = 8192
    g = torch.Generator().manual_seed(0)

    def unit():
        return types.SimpleNamespace(
            S=S, grads=[(torch.randn(2 * S, generator=g) * 1e-3).half() for _ in range(2)],
            peers=[torch.randn(S, generator=g).half()], master=torch.randn(S, generator=g) * 0.02,
            m=torch.zeros(S), v=torch.zeros(S))

    def np_of_bytes(t):
        import numpy as np
        if t.dtype == torch.float16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    units = [unit(), unit()]
    hosts = [bench.HostUnit(u, np_of_bytes) for u in units]
    per_elt = bench.sizes(cfg, "unit", "f32", 2)[1]
    assert per_elt == 34
    one = bench.cpu_baseline(cfg, hosts, per_elt, min_seconds=0.1, blocks=2)
    many = bench.cpu_baseline(cfg, hosts, per_elt, threads=4, min_seconds=0.1, blocks=36)
    assert one["cores"] == 1 and many["cores"] == 4
    for r in (one, many):
        assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0 and r["elements_per_s"] > 0
        assert r["bytes_per_shard_element"] == 34
        assert abs(r["value"] - r["elements_per_s"] * 34 / 1e9) <= 1e-3 * r["value"] + 1e-4
    assert not one["extrapolated"] and "whole units: all 2 blocks" in one["sample"]
    assert many["extrapolated"] and "extrapolated from K = 2" in many["sample"]
    assert "disjoint chunks" in many["sample"]
    # the per-step time scales the pool's pass to the step's 36 slots
    assert many["seconds_per_step"] > 0
    # the device inputs were copied before timing: the host state moved, the device state did not
    assert not (units[0].master.numpy() == hosts[0].p).all()


def test_flatten_rate_rotation_streams_past_the_last_level_cache():
    # a rotation of the flatten / unflatten rate measurements touches at least
    # four times the 256 MB cache, unless the set count is capped; a call that
    # alone exceeds that needs one set
    for nbytes in (1, 8_000_000, 78_709_760, 157_419_520, 1 << 30, 2_517_114_880, 12_460_864_000):
        k = bench.rotation(nbytes)
        assert 1 <= k <= bench.ROTATION_MAX
        assert k * nbytes >= bench.ROTATION_BYTES or k == bench.ROTATION_MAX
        assert k == 1 or (k - 1) * nbytes < bench.ROTATION_BYTES
    assert bench.ROTATION_BYTES >= 4 * (256 << 20)
    assert bench.rotation(157_419_520) == 7 and bench.rotation(6_845_104_128) == 1
