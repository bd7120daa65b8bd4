"""Synthetic FSDP-unit workloads: tensor lists and seeded input generators.

This module is shared by the tests, the benchmark and the smoke check.  It holds
none of the pipeline's arithmetic (no reduction, no optimizer, no cast of
results, no layout computation): it lists shapes and draws seeded random inputs.
Where a generated buffer is longer than the unit (the tail padding), the caller
supplies that length.

Workload shapes follow the models the pages train with FSDP: GPT-2 Large and
GPT-2 XL ("PyTorch Fully Sharded Data Parallel を使用した大規模モデル学習の加速",
section "GPT-2 でのパフォーマンス ベンチマーク"), fairseq's 13B GPT-3 ("fairseq 中的
Fully Sharded Data Parallel (FSDP) 实战指南", examples) and the 70B, 96-layer model
of "FSDP (Fully Sharded Data Parallel)", section "The Sharding Scheme".  Only the
shapes are taken; every value is synthetic.

Seeds: base seed 0; every buffer has its own generator stream seeded
``1000 * block + 10 * kind + rank`` (kinds below).  Values are drawn in fp32 and
rounded to the storage dtype by torch's round-to-nearest-even cast.
"""
from dataclasses import dataclass, field
from typing import List, Tuple

import torch

KIND_PARAM, KIND_GRAD, KIND_M, KIND_V, KIND_ZERO_MASK, KIND_OUTLIER_MASK = 0, 1, 2, 3, 4, 5

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def gpt_block(d: int, prefix: str = "") -> List[Tuple[str, Tuple[int, ...]]]:
    """A GPT-2-style transformer block in parameter order: two LayerNorms,
    fused qkv, attention projection, and a 4d MLP, each with a bias."""
    p = prefix
    return [
        (p + "ln1.w", (d,)), (p + "ln1.b", (d,)),
        (p + "qkv.w", (d, 3 * d)), (p + "qkv.b", (3 * d,)),
        (p + "proj.w", (d, d)), (p + "proj.b", (d,)),
        (p + "ln2.w", (d,)), (p + "ln2.b", (d,)),
        (p + "fc.w", (d, 4 * d)), (p + "fc.b", (4 * d,)),
        (p + "fc2.w", (4 * d, d)), (p + "fc2.b", (d,)),
    ]


def gpt2_model(d: int, n_layers: int, vocab: int, n_pos: int):
    t = [("wte", (vocab, d)), ("wpe", (n_pos, d))]
    for i in range(n_layers):
        t += gpt_block(d, "h%d." % i)
    return t


def llama_block(d: int, d_qkv: int, d_ff: int):
    """Attention (GQA-fused qkv, output) and SwiGLU MLP weights, no norms."""
    return [("qkv", (d, d_qkv)), ("o", (d, d)), ("gate", (d, d_ff)), ("up", (d, d_ff)),
            ("down", (d_ff, d))]


@dataclass
class UnitConfig:
    """One FSDP unit configuration.

    world:        N simulated data-parallel ranks
    grad_dt:      dtype of each rank's flat gradient buffer
    fp32_reduce:  reduce-scatter in fp32 (--fp32-reduce-scatter)
    compute_dt:   dtype of the compute copy that is gathered
    gathers:      all-gathers per step (2 when reshard_after_forward is on)
    blocks:       units streamed per step
    pool:         distinct units kept resident for the benchmark
    """
    name: str
    tensors: List[Tuple[str, Tuple[int, ...]]]
    world: int
    grad_dt: str
    fp32_reduce: bool
    compute_dt: str
    grad_sigma: float
    gathers: int = 1
    blocks: int = 1
    pool: int = 1
    param_sigma: float = 0.02
    mv_sigma: float = 0.0          # 0: m = v = 0; else m, v ~ |N(0, mv_sigma)|
    zero_frac: float = 0.0         # fraction of grad elements set to +0
    outlier_frac: float = 0.0      # fraction of grad elements multiplied by outlier_scale
    outlier_scale: float = 100.0
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    step: int = 1
    description: str = ""

    @property
    def numels(self) -> List[int]:
        out = []
        for _, s in self.tensors:
            n = 1
            for x in s:
                n *= x
            out.append(n)
        return out

    @property
    def shapes(self):
        return [s for _, s in self.tensors]

    @property
    def numel(self) -> int:
        return sum(self.numels)


CONFIGS = {
    "tiny": UnitConfig(
        name="tiny", tensors=[("w", (1000, 999)), ("b", (999,)), ("s", (1,))], world=2,
        grad_dt="f32", fp32_reduce=True, compute_dt="f32", grad_sigma=1e-3,
        description="3 fp32 tensors, 1,000,000 elements, N=2"),
    "gpt2-large-block": UnitConfig(
        name="gpt2-large-block", tensors=gpt_block(1280), world=2, grad_dt="f16",
        fp32_reduce=True, compute_dt="f16", grad_sigma=1e-4, blocks=36, pool=36,
        description="GPT-2 Large block d=1280 (19,677,440 elements), N=2, fp16 grads, "
                    "fp32 reduce-scatter, fp16 compute copy, 36 blocks per step"),
    "gpt2-xl-model": UnitConfig(
        name="gpt2-xl-model", tensors=gpt2_model(1600, 48, 50257, 1024), world=2,
        grad_dt="bf16", fp32_reduce=False, compute_dt="bf16", grad_sigma=1e-4,
        mv_sigma=1e-4, zero_frac=0.01,
        description="GPT-2 XL whole model as one unit (1,557,608,000 elements), N=2, "
                    "bf16 grads with 1% zeros, bf16 reduce-scatter, bf16 compute copy"),
    "gpt3-13b-block": UnitConfig(
        name="gpt3-13b-block", tensors=gpt_block(5120), world=8, grad_dt="f16",
        fp32_reduce=True, compute_dt="f16", grad_sigma=1e-4, gathers=2, blocks=40, pool=4,
        description="GPT-3 13B block d=5120 (314,639,360 elements), N=8, fp16 grads, "
                    "fp32 reduce-scatter, fp16 compute copy, 40 blocks, gathered twice"),
    "llama70b-block": UnitConfig(
        name="llama70b-block", tensors=llama_block(8192, 10240, 28672), world=8,
        grad_dt="bf16", fp32_reduce=False, compute_dt="bf16", grad_sigma=5e-5,
        outlier_frac=0.001, outlier_scale=100.0, blocks=96, pool=2,
        description="70B-shaped block (855,638,016 elements), N=8, bf16 grads with 0.1% "
                    "x100 outliers, bf16 reduce-scatter, bf16 compute copy, 96 blocks"),
}


def scaled(cfg: UnitConfig, tensors, name=None, **over) -> UnitConfig:
    """Same dtypes and distributions as `cfg` with another tensor list."""
    d = dict(cfg.__dict__)
    d.update(over)
    d["tensors"] = tensors
    d["name"] = name or (cfg.name + "-scaled")
    return UnitConfig(**d)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _seed(block: int, kind: int, rank: int) -> int:
    return 1000 * block + 10 * kind + rank


def _fill(length: int, numel: int, values: torch.Tensor, dtype: torch.dtype, device):
    out = torch.zeros(length, dtype=dtype, device=device)
    if numel:
        out[:numel] = values.to(dtype)
    return out


def param_tensors(cfg: UnitConfig, block: int = 0, device="cpu") -> List[torch.Tensor]:
    """The unit's fp32 parameters, N(0, param_sigma), as separate tensors."""
    g = _gen(_seed(block, KIND_PARAM, 0), device)
    flat = torch.randn(cfg.numel, generator=g, device=device, dtype=torch.float32) * cfg.param_sigma
    out, pos = [], 0
    for n, s in zip(cfg.numels, cfg.shapes):
        out.append(flat[pos:pos + n].clone().reshape(s))
        pos += n
    return out


def rank_grad(cfg: UnitConfig, block: int, rank: int, length: int, device="cpu") -> torch.Tensor:
    """Rank `rank`'s flat gradient of `length` >= numel elements: N(0, grad_sigma)
    over the unit, with the configured zeros and outliers, rounded to grad_dt;
    +0 beyond the unit."""
    P = cfg.numel
    g = _gen(_seed(block, KIND_GRAD, rank), device)
    x = torch.randn(P, generator=g, device=device, dtype=torch.float32) * cfg.grad_sigma
    if cfg.outlier_frac > 0:
        mg = _gen(_seed(block, KIND_OUTLIER_MASK, rank), device)
        mask = torch.rand(P, generator=mg, device=device) < cfg.outlier_frac
        x = torch.where(mask, x * cfg.outlier_scale, x)
    if cfg.zero_frac > 0:
        zg = _gen(_seed(block, KIND_ZERO_MASK, rank), device)
        mask = torch.rand(P, generator=zg, device=device) < cfg.zero_frac
        x = torch.where(mask, torch.zeros_like(x), x)
    return _fill(length, P, x, TORCH_DTYPE[cfg.grad_dt], device)


def rank_grads(cfg: UnitConfig, block: int, length: int, device="cpu") -> torch.Tensor:
    """Every simulated rank's flat gradient of the unit as the rows of one
    [world, length] view: row q holds rank_grad(cfg, block, q, length).  One
    allocation puts the N gradient streams at a fixed row stride from each other,
    whatever the allocator does with separate buffers.  The stride is length
    rounded up to 64 elements, so every row starts on a 128-byte line and keeps
    the 16-byte alignment of the kernels' vector path for any world size and
    length (a stride of an odd length of 16-bit elements would leave every other
    row 2-byte aligned, and the kernels would take their per-element path)."""
    stride = (length + 63) // 64 * 64
    out = torch.empty((cfg.world, stride), dtype=TORCH_DTYPE[cfg.grad_dt], device=device)[:, :length]
    for q in range(cfg.world):
        out[q].copy_(rank_grad(cfg, block, q, length, device))
    return out


def moments(cfg: UnitConfig, block: int, begin: int, count: int, numel_limit: int, device="cpu"):
    """fp32 m and v for positions [begin, begin+count) of the (padded) flat unit:
    zero, or |N(0, mv_sigma)| inside the unit and +0 in the padding."""
    if cfg.mv_sigma == 0.0:
        z = torch.zeros(count, dtype=torch.float32, device=device)
        return z, z.clone()
    out = []
    for kind in (KIND_M, KIND_V):
        g = _gen(_seed(block, kind, 0), device)
        x = (torch.randn(numel_limit, generator=g, device=device, dtype=torch.float32)
             * cfg.mv_sigma).abs()
        buf = torch.zeros(count, dtype=torch.float32, device=device)
        hi = min(begin + count, numel_limit)
        if hi > begin:
            buf[:hi - begin] = x[begin:hi]
        out.append(buf)
    return out[0], out[1]
