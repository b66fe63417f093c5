"""Seeded synthetic inputs for the segmented-gather multi-LoRA path.

This module only draws random inputs; it holds none of the method's
arithmetic, so both the HIP path and the CPU oracle can be fed from it
without sharing any computation.

Recipe (one ``torch.Generator('cpu')`` per workload, seeded with the
workload's index; draw order: mapping, then per layer x, A slices, B slices,
bias slices, y0; normal values are drawn in float32 and rounded to bfloat16):

* ``tiny``     N=64,    H=256   -> [256],              r=8,   max_loras=3,
  ids iid uniform over {-1,0,1,2}, scale 0.5.
* ``decode``   N=256,   H=4096  -> [4096,1024,1024],   r=16,  max_loras=32,
  ids iid uniform 0..31, then round(0.10 N) positions set to -1, scale 1.0.
* ``prefill``  N=8192,  H=4096  -> [4096,1024,1024],   r=64,  max_loras=8,
  16 contiguous runs of 512 tokens, each run one id uniform 0..7, per-slice
  bias ~N(0, 0.01), scale 0.25.
* ``zipf``     N=4096, two layers sharing one mapping: gate/up
  H=4096 -> [14336,14336] and down H=14336 -> [4096] (fresh x), r=32,
  max_loras=64, ids iid from a Zipf law truncated to 0..63 with
  p(k) proportional to (k+1)^-1.1, then round(0.05 N) positions set to -1,
  scale 0.5.
* ``large``    N=16384, H=8192  -> [8192,1024,1024],   r=128, max_loras=128,
  ids iid uniform 0..127 (tokens interleaved), then round(0.20 N) positions
  set to -1, scale 0.125, weights ~N(0, 0.01).
* ``large_nolora``  the ``large`` shapes with every id -1 (seed 5).
* ``logits``   N=256 prompts (one sampled position each), H=4096 -> one
  vocab-wide slice [128256], r=16, max_loras=32, ids iid uniform 0..31, then
  round(0.10 N) positions set to -1, scale 1.0 (the logits path: shrink +
  expand over the per-prompt mapping).
* ``embedding`` N=8192, expand only: input [1][N][16] fp32 ~N(0,1) -> one
  slice [4096], r=16, max_loras=32, ids iid uniform 0..31, then round(0.10 N)
  positions set to -1 (the embedding path).

x and y0 are ~N(0,1); weights ~N(0,0.02) unless stated; sigma is the
standard deviation.  "p % set to -1" picks exactly round(p N) positions with
a seeded permutation.

An expand-only layer draws, in order, its fp32 input ``x`` [1][N][r], the
B slices, the bias slices (if any) and y0; it has no A.

Storage layouts (the library's and the oracle's common input contract):
``x`` [N][H] row-major (expand-only layers: fp32 [1][N][r]);
``A_i`` [max_loras][r][H]; ``B_i`` [max_loras][O_i][r];
``bias_i`` [max_loras][O_i]; ``y0`` [N][sum O_i]; shrink buffer [S][N][r] fp32.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import torch


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    hidden: int
    slices: tuple
    rank: int
    scale: float
    sigma_w: float = 0.02
    sigma_bias: Optional[float] = None
    expand_only: bool = False    # no shrink: x is the fp32 expand input [1][N][r]


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    name: str
    seed: int
    num_tokens: int
    max_loras: int
    mapping_kind: str
    layers: tuple
    neg_fraction: float = 0.0
    description: str = ""


WORKLOADS: Dict[str, WorkloadSpec] = {
    "tiny": WorkloadSpec(
        "tiny", 0, 64, 3, "uniform_with_neg",
        (LayerSpec(256, (256,), 8, 0.5),),
        description="N=64 H=256 r=8 max_loras=3 1 slice, ids uniform {-1,0,1,2}"),
    "decode": WorkloadSpec(
        "decode", 1, 256, 32, "uniform", (LayerSpec(4096, (4096, 1024, 1024), 16, 1.0),),
        neg_fraction=0.10,
        description="N=256 H=4096 r=16 max_loras=32 qkv 4096/1024/1024, 10% -1"),
    "prefill": WorkloadSpec(
        "prefill", 2, 8192, 8, "runs",
        (LayerSpec(4096, (4096, 1024, 1024), 64, 0.25, sigma_bias=0.01),),
        description="N=8192 as 16 runs of 512, ids 0..7, H=4096 r=64 qkv + bias"),
    "zipf": WorkloadSpec(
        "zipf", 3, 4096, 64, "zipf",
        (LayerSpec(4096, (14336, 14336), 32, 0.5), LayerSpec(14336, (4096,), 32, 0.5)),
        neg_fraction=0.05,
        description="N=4096 Zipf(1.1) over 64 ids, 5% -1; gate/up 4096->2x14336, down 14336->4096, r=32"),
    "large": WorkloadSpec(
        "large", 4, 16384, 128, "uniform",
        (LayerSpec(8192, (8192, 1024, 1024), 128, 0.125, sigma_w=0.01),),
        neg_fraction=0.20,
        description="N=16384 H=8192 r=128 max_loras=128 qkv 8192/1024/1024, 20% -1"),
    "large_nolora": WorkloadSpec(
        "large_nolora", 5, 16384, 128, "all_neg",
        (LayerSpec(8192, (8192, 1024, 1024), 128, 0.125, sigma_w=0.01),),
        description="large shapes, every id -1"),
    "logits": WorkloadSpec(
        "logits", 6, 256, 32, "uniform", (LayerSpec(4096, (128256,), 16, 1.0),),
        neg_fraction=0.10,
        description="logits path: 256 prompts, H=4096 -> vocab 128256, r=16, max_loras=32, 10% -1"),
    "embedding": WorkloadSpec(
        "embedding", 7, 8192, 32, "uniform", (LayerSpec(16, (4096,), 16, 1.0, expand_only=True),),
        neg_fraction=0.10,
        description="embedding path: expand only, N=8192, input [N][16] fp32 -> 4096, max_loras=32, 10% -1"),
}


def _normal_bf16(gen: torch.Generator, shape, sigma: float) -> torch.Tensor:
    t = torch.randn(shape, generator=gen, dtype=torch.float32)
    if sigma != 1.0:
        t.mul_(sigma)
    return t.to(torch.bfloat16)


def _set_negative(gen: torch.Generator, mapping: torch.Tensor, fraction: float) -> None:
    n = mapping.numel()
    k = int(round(fraction * n))
    if k:
        pos = torch.randperm(n, generator=gen)[:k]
        mapping[pos] = -1


def make_mapping(spec: WorkloadSpec, gen: torch.Generator) -> torch.Tensor:
    n, ml = spec.num_tokens, spec.max_loras
    kind = spec.mapping_kind
    if kind == "uniform_with_neg":
        m = torch.randint(-1, ml, (n,), generator=gen, dtype=torch.int64)
    elif kind == "uniform":
        m = torch.randint(0, ml, (n,), generator=gen, dtype=torch.int64)
    elif kind == "runs":
        runs = 16
        ids = torch.randint(0, ml, (runs,), generator=gen, dtype=torch.int64)
        lens = torch.tensor([n // runs + (1 if i < n % runs else 0) for i in range(runs)])
        m = ids.repeat_interleave(lens)
    elif kind == "zipf":
        p = torch.arange(1, ml + 1, dtype=torch.float64).pow(-1.1)
        m = torch.multinomial(p / p.sum(), n, replacement=True, generator=gen)
    elif kind == "all_neg":
        m = torch.full((n,), -1, dtype=torch.int64)
    else:
        raise ValueError(kind)
    m = m.to(torch.int32).contiguous()
    _set_negative(gen, m, spec.neg_fraction)
    return m


@dataclasses.dataclass
class Layer:
    spec: LayerSpec
    x: torch.Tensor                 # bf16 [N][H]; expand-only layers: fp32 [1][N][r]
    lora_a: List[torch.Tensor]      # bf16 [max_loras][r][H] per slice (none if expand-only)
    lora_b: List[torch.Tensor]      # bf16 [max_loras][O_i][r] per slice
    bias: Optional[List[torch.Tensor]]  # bf16 [max_loras][O_i] per slice, or None
    y0: torch.Tensor                # bf16 [N][sum O_i]


@dataclasses.dataclass
class Workload:
    spec: WorkloadSpec
    mapping: torch.Tensor           # int32 [N]
    layers: List[Layer]


def make_layer(spec: LayerSpec, n: int, max_loras: int, gen: torch.Generator) -> Layer:
    if spec.expand_only:
        x = torch.randn((1, n, spec.rank), generator=gen, dtype=torch.float32)
        a = []
    else:
        x = _normal_bf16(gen, (n, spec.hidden), 1.0)
        a = [_normal_bf16(gen, (max_loras, spec.rank, spec.hidden), spec.sigma_w) for _ in spec.slices]
    b = [_normal_bf16(gen, (max_loras, w, spec.rank), spec.sigma_w) for w in spec.slices]
    bias = None
    if spec.sigma_bias is not None:
        bias = [_normal_bf16(gen, (max_loras, w), spec.sigma_bias) for w in spec.slices]
    y0 = _normal_bf16(gen, (n, sum(spec.slices)), 1.0)
    return Layer(spec, x, a, b, bias, y0)


def make_workload(name: str, seed: Optional[int] = None, num_tokens: Optional[int] = None) -> Workload:
    """Build one workload's inputs on the CPU.

    ``num_tokens`` overrides N (used to make small cases of a workload's
    shapes); ``seed`` overrides the workload's own seed.
    """
    spec = WORKLOADS[name]
    if num_tokens is not None:
        spec = dataclasses.replace(spec, num_tokens=num_tokens)
    gen = torch.Generator("cpu")
    gen.manual_seed(spec.seed if seed is None else seed)
    mapping = make_mapping(spec, gen)
    layers = [make_layer(ls, spec.num_tokens, spec.max_loras, gen) for ls in spec.layers]
    return Workload(spec, mapping, layers)


def make_buffer(gen: torch.Generator, num_slices: int, n: int, rank: int, sigma: float) -> torch.Tensor:
    """A synthetic fp32 shrink buffer [S][N][r] ~N(0, sigma), used to drive
    the expand step on its own."""
    return torch.randn((num_slices, n, rank), generator=gen, dtype=torch.float32).mul_(sigma)


def random_case(seed: int, n: int, hidden: int, slices, rank: int, max_loras: int,
                neg_fraction: float = 0.25, bias: bool = False, scale: float = 0.5,
                sigma_w: float = 0.02) -> Workload:
    """A small random case of arbitrary shape (ids iid uniform in
    [-1, max_loras) after a negative fraction is forced)."""
    spec = WorkloadSpec("random", seed, n, max_loras, "uniform",
                        (LayerSpec(hidden, tuple(slices), rank, scale, sigma_w,
                                   0.01 if bias else None),),
                        neg_fraction=neg_fraction)
    gen = torch.Generator("cpu")
    gen.manual_seed(seed)
    mapping = make_mapping(spec, gen)
    layers = [make_layer(spec.layers[0], n, max_loras, gen)]
    return Workload(spec, mapping, layers)


def bf16_bits(t: torch.Tensor):
    """Raw bfloat16 bit patterns of a CPU tensor as a numpy uint16 array."""
    import numpy as np
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
