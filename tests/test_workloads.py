"""Workload table and seeded generators.

Unit sizes are closed forms of the listed shapes: a GPT-2 block of width d holds
12 d^2 + 13 d parameters; GPT-2 XL adds a 50257 x 1600 token embedding and a
1024 x 1600 position embedding to 48 blocks; the 70B-shaped block is
8192 x (10240 + 8192 + 3 * 28672)."""
import torch

from workloads import CONFIGS, moments, param_tensors, rank_grad, rank_grads, scaled, gpt_block


def test_unit_sizes():
    blk = lambda d: 12 * d * d + 13 * d  # noqa: E731
    assert CONFIGS["tiny"].numel == 1_000_000
    assert CONFIGS["gpt2-large-block"].numel == blk(1280) == 19_677_440
    assert CONFIGS["gpt2-xl-model"].numel == 50257 * 1600 + 1024 * 1600 + 48 * blk(1600) == 1_557_608_000
    assert CONFIGS["gpt3-13b-block"].numel == blk(5120) == 314_639_360
    assert CONFIGS["llama70b-block"].numel == 8192 * (10240 + 8192 + 3 * 28672) == 855_638_016
    assert len(CONFIGS["gpt2-xl-model"].tensors) == 2 + 48 * 12


def test_generators_are_seeded_and_padded():
    cfg = scaled(CONFIGS["llama70b-block"], gpt_block(64), name="t")
    a = rank_grad(cfg, 3, 5, cfg.numel + 3)
    b = rank_grad(cfg, 3, 5, cfg.numel + 3)
    c = rank_grad(cfg, 3, 4, cfg.numel + 3)
    assert a.dtype == torch.bfloat16 and torch.equal(a, b) and not torch.equal(a, c)
    assert torch.count_nonzero(a[cfg.numel:]) == 0
    p1 = param_tensors(cfg, 0)
    assert [tuple(t.shape) for t in p1] == [s for s in cfg.shapes]


def test_distributions():
    cfg = scaled(CONFIGS["gpt2-xl-model"], [("w", (400, 1000))], name="t")
    g = rank_grad(cfg, 0, 0, cfg.numel).float()
    zero = (g == 0).float().mean().item()
    assert 0.008 < zero < 0.012
    assert abs(g[g != 0].std().item() / 1e-4 - 1) < 0.02
    m, v = moments(cfg, 0, 0, cfg.numel + 2, cfg.numel)
    assert (m[:cfg.numel] >= 0).all() and m[cfg.numel:].count_nonzero() == 0
    cfg5 = scaled(CONFIGS["llama70b-block"], [("w", (1000, 1000))], name="t5")
    g5 = rank_grad(cfg5, 0, 0, cfg5.numel).float()
    frac = (g5.abs() > 20 * 5e-5).float().mean().item()
    assert 0.0007 < frac < 0.0013


def test_stacked_gradients_are_the_ranks_gradients():
    # one [world, length] buffer whose row q is rank q's gradient, byte for byte
    cfg = scaled(CONFIGS["gpt3-13b-block"], gpt_block(32) + [("odd", (3,))], name="t", world=3)
    length = cfg.numel + 2
    st = rank_grads(cfg, 2, length)
    assert st.shape == (3, length) and st.dtype == torch.float16
    for q in range(3):
        assert st[q].is_contiguous()
        assert torch.equal(st[q].view(torch.int16), rank_grad(cfg, 2, q, length).view(torch.int16))
    # rows start on 128-byte lines whatever the length: here length is odd
    assert length % 2 == 1 and st.stride(0) == (length + 63) // 64 * 64
    assert all((st[q].data_ptr() - st.data_ptr()) % 128 == 0 for q in range(3))
    # a length that is already a whole number of lines keeps the rows back to back
    whole = (cfg.numel + 63) // 64 * 64
    st2 = rank_grads(cfg, 2, whole)
    assert st2.stride(0) == whole and st2.is_contiguous()
