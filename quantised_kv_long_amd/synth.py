"""Seeded synthetic inputs and the workload shapes they follow.

This module holds no arithmetic of the method (no quantisation, no attention):
it only draws seeded random fp16 tensors and builds the structured inputs the
workloads call for (outlier channels, a planted needle key, ragged lengths).
It is shared by the tests, the benchmark and the oracle checks, which all
receive the same bytes.

Workload shapes follow the pages' models:
  * HAL #582 "per-layer KV compression study": vehicle with 48 layers, 8 KV
    heads, head_dim 128 (section 0 header), q8_0K/q4_0V default tier
    (section 4), contexts 64k-128k (section 3b) and up to 1M (section 1);
  * qwisp issue #168: full-attention layer [2, ctx, 256] (2 KV heads,
    head_dim 256) of a hybrid model, contexts up to 262,144.
The query-head counts (40 and 16) and the value distributions are this
project's choices; they are documented with each workload.

Random stream: every tensor is drawn on the device with torch's Philox
generator seeded with ``seed_for(workload_seed, layer, tensor, step)``, in
fp32 from N(0, 1), then rounded to fp16 (round to nearest even).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "k_new": 3, "v_new": 4, "aux": 5}


def seed_for(base: int, layer: int = 0, tensor: str = "q", step: int = 0) -> int:
    return (base * 1_000_003 + layer * 10_007 + TENSOR_IDS[tensor] * 101 + step) % (2**62)


def normal_f16(shape, seed: int, device="cuda", scale: float = 1.0) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale
    return x.to(torch.float16)


def outlier_channels(D: int, seed: int, frac: float = 0.01) -> list[int]:
    """round(frac * D) distinct channel indices (the same for every token)."""
    n = max(1, round(frac * D))
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return sorted(torch.randperm(D, generator=g)[:n].tolist())


def ragged_lengths(B: int, lo: int, hi: int, seed: int) -> list[int]:
    """B integers uniform in [lo, hi]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.randint(lo, hi + 1, (B,), generator=g).tolist()


def needle_row(q_head: torch.Tensor, seed: int, cosine: float = 0.9) -> torch.Tensor:
    """A key row with the given cosine to ``q_head`` and norm sqrt(D):
    sqrt(D) * (c * u + sqrt(1 - c^2) * r), u = q / |q|, r a seeded unit vector
    orthogonal to u.  Returned as fp16 on q_head's device."""
    q = q_head.double().flatten()
    D = q.numel()
    u = q / q.norm()
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    r = torch.randn(D, generator=g, dtype=torch.float64).to(q.device)
    r = r - (r @ u) * u
    r = r / r.norm()
    k = math.sqrt(D) * (cosine * u + math.sqrt(1.0 - cosine * cosine) * r)
    return k.to(torch.float16)


@dataclass
class Workload:
    name: str
    description: str
    layers: int
    B: int
    Hq: int
    Hkv: int
    D: int
    ctx: int                       # context after the appended token (max for ragged)
    arms: list[tuple[str, str]]
    seed: int
    split_tokens: int
    k_outlier_frac: float = 0.0    # fraction of K channels scaled x8 (0 = none)
    needle: bool = False
    ragged: tuple[int, int] | None = None   # (lo, hi) lengths, uniform
    variants: list["Workload"] = field(default_factory=list)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def lengths(self) -> list[int]:
        if self.ragged is None:
            return [self.ctx] * self.B
        return ragged_lengths(self.B, self.ragged[0], self.ragged[1], self.seed)


WORKLOADS = {
    "gqa5_d128_ctx4k": Workload(
        "gqa5_d128_ctx4k",
        "one layer, batch 1, 40 query / 8 KV heads, head_dim 128, ctx 4096, K q8_0 + V q4_0, "
        "K, V, Q ~ N(0,1)",
        layers=1, B=1, Hq=40, Hkv=8, D=128, ctx=4096, arms=[("q8_0", "q4_0")], seed=1001,
        split_tokens=128),
    "hybrid_d256_ctx32k": Workload(
        "hybrid_d256_ctx32k",
        "hybrid-model full-attention layer: 16 query / 2 KV heads, head_dim 256, ctx 32768, "
        "batch 1; K ~ N(0,1) with 1% of channels scaled x8, V, Q ~ N(0,1)",
        layers=1, B=1, Hq=16, Hkv=2, D=256, ctx=32768, arms=[("f16", "f16"), ("q8_0", "q8_0")],
        seed=1002, split_tokens=256, k_outlier_frac=0.01),
    "stack48_d128_ctx64k": Workload(
        "stack48_d128_ctx64k",
        "48-layer decode stack: 40 query / 8 KV heads, head_dim 128, ctx 65536, batch 1; per "
        "layer append one token then attend; N(0,1)",
        layers=48, B=1, Hq=40, Hkv=8, D=128, ctx=65536,
        arms=[("f16", "f16"), ("q8_0", "q4_0"), ("q4_0", "q4_0")], seed=1003, split_tokens=1024),
    "stack48_d128_ctx64k_types": Workload(
        "stack48_d128_ctx64k_types",
        "the 48-layer 64k decode stack of stack48_d128_ctx64k with the further scalar types: "
        "the pages' served pairs with q4_1 / q5_0 / q5_1 / q6_0 and the tier ladder's q5_1 K + "
        "q4_0 V, q8_0 K + q4_0 V for reference; N(0,1)",
        layers=48, B=1, Hq=40, Hkv=8, D=128, ctx=65536,
        arms=[("q8_0", "q4_0"), ("q5_1", "q4_0"), ("q4_1", "q4_1"), ("q5_0", "q5_0"), ("q5_1", "q5_1"),
              ("q6_0", "q6_0"), ("q6_0", "q4_0"), ("q8_0", "q5_0"), ("q8_0", "q6_0")],
        seed=1003, split_tokens=1024),
    "long_d128_ctx256k": Workload(
        "long_d128_ctx256k",
        "one layer, 40 query / 8 KV heads, head_dim 128, ctx 262144, batch 1; keys N(0,1) with "
        "one planted needle row of cosine 0.9 to the group's first query head",
        layers=1, B=1, Hq=40, Hkv=8, D=128, ctx=262144, arms=[("q8_0", "q4_0"), ("q4_0", "q4_0")],
        seed=1004, split_tokens=4096, needle=True),
    "batch16_ragged": Workload(
        "batch16_ragged",
        "16 sequences, ctx uniform in [16384, 131072], 40 query / 8 KV heads, head_dim 128; "
        "N(0,1)",
        layers=1, B=16, Hq=40, Hkv=8, D=128, ctx=131072, arms=[("q4_0", "q4_0"), ("q8_0", "q4_0")],
        seed=1005, split_tokens=2048, ragged=(16384, 131072)),
    "batch16_ragged_d512": Workload(
        "batch16_ragged_d512",
        "16 sequences, ctx uniform in [16384, 131072], 16 query / 2 KV heads, head_dim 512; N(0,1)",
        layers=1, B=16, Hq=16, Hkv=2, D=512, ctx=131072, arms=[("q4_0", "q4_0"), ("q8_0", "q4_0")],
        seed=1006, split_tokens=1024, ragged=(16384, 131072)),
}
