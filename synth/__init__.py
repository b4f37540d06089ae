"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no arithmetic of the method: it only draws N(0, 1) tensors
from a seeded torch generator, rounds them to the working dtype, and describes
the five workloads (shapes, dtype, frequency-scaling parameters).  Both the HIP
path and the fp64 oracle consume the very same tensors: the oracle gets a host
copy of what was uploaded (bf16 values upcast exactly to fp64).

Seeding: tensor ``tid`` (q=0, k=1, v=2) of workload ``seed`` uses
``seed * 1_000_003 + tid * 65_537``.  A generator on the CPU and one on the GPU
give different streams for the same seed; every comparison therefore feeds the
oracle from the tensor actually handed to the kernel, never from a re-draw.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

Q_ID, K_ID, V_ID, DO_ID = 0, 1, 2, 3   # dO: upstream gradient of the backward tests

# rope method codes, same numbering as the C header
NONE, PI, NTK, YARN = 0, 1, 2, 3


def seed_for(seed: int, tid: int) -> int:
    return seed * 1_000_003 + tid * 65_537


def randn(shape, dtype: torch.dtype, seed: int, tid: int, device="cpu") -> torch.Tensor:
    """N(0,1) draws in fp32, rounded (round-to-nearest-even) to ``dtype``."""
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(seed, tid))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    return x if dtype == torch.float32 else x.to(dtype)


@dataclass(frozen=True)
class Rope:
    """Frequency-scaling parameters of one workload."""
    method: int = NONE
    base: float = 10000.0
    s: float = 1.0          # scale factor L'/L
    L: float = 0.0          # training length (YaRN only)
    alpha: float = 1.0      # NTK-by-parts lower ramp bound (YaRN only)
    beta: float = 32.0      # NTK-by-parts upper ramp bound (YaRN only)


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    N: int
    D: int
    dtype: torch.dtype
    rope: Rope
    kind: str = "prefill"            # prefill | ring | decode
    chunks: int = 1                  # ring: K/V chunks merged by log-sum-exp
    splits: int = 1                  # decode: KV blocks per sequence
    causal: bool = True
    note: str = field(default="", compare=False)

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 1, 1, 1, 512, 64, torch.float32, Rope(NONE, 10000.0),
                   note="B=1 H=1 N=512 D=64 fp32 causal, plain RoPE base 1e4"),
    "gqa_8k_bf16": Workload("gqa_8k_bf16", 2, 1, 32, 8, 8192, 128, torch.bfloat16, Rope(NONE, 500000.0),
                   note="GQA 32/8 D=128 N=8192 bf16 causal, RoPE base 5e5 unscaled"),
    "yarn_32k_bf16": Workload("yarn_32k_bf16", 3, 1, 32, 8, 32768, 128, torch.bfloat16,
                   Rope(YARN, 10000.0, 16.0, 2048.0, 1.0, 32.0),
                   note="GQA 32/8 D=128 N=32768 bf16 causal, YaRN base 1e4 L=2048 s=16 a=1 b=32"),
    "ntk_128k_ring_bf16": Workload("ntk_128k_ring_bf16", 4, 1, 32, 8, 131072, 128, torch.bfloat16,
                   Rope(NTK, 10000.0, 16.0), kind="ring", chunks=8,
                   note="GQA 32/8 D=128 N=131072 bf16 causal, NTK 8K->128K, 8 K/V chunks merged by LSE"),
    "decode_128k_bf16": Workload("decode_128k_bf16", 5, 16, 32, 8, 131072, 128, torch.bfloat16,
                   Rope(PI, 10000.0, 16.0), kind="decode", splits=64,
                   note="decode B=16 GQA 32/8 D=128, 131072-position bf16 cache, PI s=16, 64 splits"),
}
