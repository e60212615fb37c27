"""Seeded synthetic inputs for the quantized MoE layer.

This module only draws random numbers. It holds none of the layer's arithmetic:
no packing, no unpacking, no dequantization, no routing. Both the CPU oracle
(``oracle/``) and the GPU library consume what it returns.

Weight codes are drawn as uniform random bytes. For every packing used here
(INT4 two per byte, INT3 eight per three bytes, INT2 four per byte) each code's
bits are independent uniform bits, so uniform bytes give uniform codes.

Draw order for one layer instance (fixed, so a seed reproduces everything):
sequence lengths, Zipf permutation, router logits, activations, then the
weights (fc1 codes, fc1 scales, fc2 codes, fc2 scales).

Shapes follow the Qwen3-30B-A3B expert layer the pages measure (hidden 2048,
inter 768, 128 experts, top-8; "[CUDA/CPU] Add AVX2 INT4 cold-expert kernel ..."
page, "End-to-End 48-Layer Qwen3-30B-A3B" table) plus a tiny layer for checks.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch


@dataclass(frozen=True)
class LayerSpec:
    hidden: int
    inter: int
    num_experts: int
    top_k: int
    bits: int
    block_size: int
    zero_point: int
    scale_c: float          # scales = fp16(|N(0,1)| * scale_c + 1e-3)
    act_dtype: str          # "f32", "bf16" or "f16"

    @property
    def fc1_rows(self) -> int:
        return 2 * self.inter

    def row_bytes(self, k: int) -> int:
        return k * self.bits // 8


@dataclass
class LayerWeights:
    fc1_codes: np.ndarray   # uint8 [E, 2I, H*bits/8]
    fc1_scales: np.ndarray  # float16 [E, 2I, H/bs]
    fc2_codes: np.ndarray   # uint8 [E, H, I*bits/8]
    fc2_scales: np.ndarray  # float16 [E, H, I/bs]


@dataclass
class Tokens:
    x: torch.Tensor         # [T, H] activation dtype (CPU)
    logits: torch.Tensor    # [T, E] activation dtype (CPU)
    seq_lens: List[int] = field(default_factory=list)


TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}

# The five workloads. Names say what they are.
TINY = LayerSpec(hidden=64, inter=32, num_experts=4, top_k=2, bits=4,
                 block_size=32, zero_point=8, scale_c=0.05, act_dtype="f32")
QWEN3_INT4 = LayerSpec(hidden=2048, inter=768, num_experts=128, top_k=8, bits=4,
                       block_size=32, zero_point=8, scale_c=0.02, act_dtype="bf16")
QWEN3_INT3 = LayerSpec(hidden=2048, inter=768, num_experts=128, top_k=8, bits=3,
                       block_size=64, zero_point=4, scale_c=0.03, act_dtype="bf16")
QWEN3_INT2 = LayerSpec(hidden=2048, inter=768, num_experts=128, top_k=8, bits=2,
                       block_size=32, zero_point=2, scale_c=0.02, act_dtype="bf16")


def spec_with(base: LayerSpec, **kw) -> LayerSpec:
    d = dict(base.__dict__)
    d.update(kw)
    return LayerSpec(**d)


def draw_weights(spec: LayerSpec, rng: np.random.Generator) -> LayerWeights:
    E, H, I, bs = spec.num_experts, spec.hidden, spec.inter, spec.block_size
    c = spec.scale_c

    def scales(shape):
        return (np.abs(rng.standard_normal(shape)) * c + 1e-3).astype(np.float16)

    fc1_codes = rng.integers(0, 256, size=(E, 2 * I, spec.row_bytes(H)), dtype=np.uint8)
    fc1_scales = scales((E, 2 * I, H // bs))
    fc2_codes = rng.integers(0, 256, size=(E, H, spec.row_bytes(I)), dtype=np.uint8)
    fc2_scales = scales((E, H, I // bs))
    return LayerWeights(fc1_codes, fc1_scales, fc2_codes, fc2_scales)


def draw_seq_lens(total: int, nseq: int, rng: np.random.Generator) -> List[int]:
    """A uniform random composition of ``total`` into ``nseq`` positive parts:
    nseq-1 distinct cut points drawn from 1..total-1, sorted."""
    if nseq <= 1:
        return [total]
    cuts = np.sort(rng.choice(np.arange(1, total), size=nseq - 1, replace=False))
    edges = np.concatenate([[0], cuts, [total]])
    return [int(v) for v in np.diff(edges)]


def zipf_bias(num_experts: int, s: float, rng: np.random.Generator) -> np.ndarray:
    """Per-expert logit bias 1.5*ln(p_rank) with p_r = r^-s / sum r'^-s and the
    rank order a seeded permutation of the experts (fp64)."""
    perm = rng.permutation(num_experts)          # perm[r-1] = expert of rank r
    ranks = np.arange(1, num_experts + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    bias = np.empty(num_experts, dtype=np.float64)
    bias[perm] = 1.5 * np.log(p)
    return bias


def draw_tokens(spec: LayerSpec, T: int, rng: np.random.Generator, *, nseq: int = 1,
                zipf_s: Optional[float] = None) -> Tokens:
    seq_lens = draw_seq_lens(T, nseq, rng) if T > 0 else []
    bias = zipf_bias(spec.num_experts, zipf_s, rng) if zipf_s is not None else None
    logits64 = rng.standard_normal((T, spec.num_experts))
    if bias is not None:
        logits64 = logits64 + bias[None, :]
    x64 = rng.standard_normal((T, spec.hidden))
    dt = TORCH_DTYPE[spec.act_dtype]
    # one rounding from fp64 to the stored activation dtype
    logits = torch.from_numpy(logits64).to(dt)
    x = torch.from_numpy(x64).to(dt)
    return Tokens(x=x, logits=logits, seq_lens=seq_lens)


@dataclass
class Workload:
    name: str
    spec: LayerSpec
    tokens: Tokens
    weights: LayerWeights


def make_workload(name: str, T: Optional[int] = None, seed: Optional[int] = None,
                  layer: int = 0) -> Workload:
    """Build one named workload.

    tiny      T=4 fp32 INT4 bs32 layer, H=64, E=4, top-2, I=32 (seed 1)
    decode    Qwen3-30B-A3B-shaped INT4 bs32 layer, T=1 or 4, uniform routing (seed 2)
    prefill   same layer, T=8192 packed from 16 sequences, Zipf(1.1)-biased logits (seed 3)
    int3      raw INT3 bs64 layer, T=4 decode or T=2048 packed prefill (seed 4)
    stack     one layer of the 48-layer INT2 bs32 stack, Zipf routing per layer (seed 5+layer)
    """
    if name == "tiny":
        spec, T, seed0, nseq, zipf = TINY, 4 if T is None else T, 1, 1, None
    elif name == "decode":
        spec, T, seed0, nseq, zipf = QWEN3_INT4, 4 if T is None else T, 2, 1, None
    elif name == "prefill":
        spec, T, seed0, nseq, zipf = QWEN3_INT4, 8192 if T is None else T, 3, 16, 1.1
    elif name == "int3":
        spec, T, seed0 = QWEN3_INT3, 4 if T is None else T, 4
        nseq, zipf = (8 if T > 4 else 1), None
    elif name == "stack":
        spec, T, seed0, zipf = QWEN3_INT2, 32768 if T is None else T, 5 + layer, 1.1
        nseq = 16 if T > 16 else 1
    else:
        raise ValueError(f"unknown workload {name!r}")
    if seed is not None:
        seed0 = seed
    nseq = min(nseq, max(T, 1))
    rng = np.random.default_rng(seed0)
    tokens = draw_tokens(spec, T, rng, nseq=nseq, zipf_s=zipf)
    weights = draw_weights(spec, rng)
    return Workload(name=name, spec=spec, tokens=tokens, weights=weights)


def make_layer(spec: LayerSpec, T: int, seed: int, *, nseq: int = 1,
               zipf_s: Optional[float] = None) -> Workload:
    """A workload for an arbitrary layer spec (used for format sweeps)."""
    rng = np.random.default_rng(seed)
    tokens = draw_tokens(spec, T, rng, nseq=min(nseq, max(T, 1)), zipf_s=zipf_s)
    weights = draw_weights(spec, rng)
    return Workload(name="custom", spec=spec, tokens=tokens, weights=weights)
