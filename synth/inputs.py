"""Seeded workload generator (no attention arithmetic lives here).

The five workloads are the pages' shapes: the Wan2.2 VAE mid-block attention
(one head per latent frame over 44x78 = 3432 positions, 1024 channels, scale
1/32; FastVideo wan22_vae_decode attn.cu, header comment) at 1, 4 and 31
frames, a 13x22 single-head case at d = 256, and the Blackwell FMHA example's
4 x 1024 x 8 x 64 shape with and without the causal mask (cuDNN
native_sparse_attention fmha.py, module docstring).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    d: int
    scale: float
    causal: bool
    seed: int

    @property
    def shape(self):
        return (self.B, self.H, self.L, self.d)

    def flops(self) -> int:
        """Two contractions at 2 FLOP per multiply-add over the pairs computed.

        Unmasked: 4*B*H*L*L*d.  Causal: only the L*(L+1)/2 allowed pairs.
        """
        pairs = self.L * (self.L + 1) // 2 if self.causal else self.L * self.L
        return 4 * self.B * self.H * pairs * self.d

    def io_bytes(self) -> int:
        """q, k, v read once and out written once, bf16."""
        return 4 * self.B * self.H * self.L * self.d * 2


WORKLOADS = {
    "tiny_d256": Workload("tiny_d256", 1, 1, 286, 256, 1.0 / 16, False, 1),
    "mha_d64": Workload("mha_d64", 4, 8, 1024, 64, 1.0 / 8, False, 2),
    "mha_d64_causal": Workload("mha_d64_causal", 4, 8, 1024, 64, 1.0 / 8, True, 2),
    "wan_1frame": Workload("wan_1frame", 1, 1, 3432, 1024, 1.0 / 32, False, 3),
    "wan_4frame": Workload("wan_4frame", 4, 1, 3432, 1024, 1.0 / 32, False, 4),
    "wan_31frame": Workload("wan_31frame", 31, 1, 3432, 1024, 1.0 / 32, False, 5),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def make_qkv(B: int, H: int, L: int, d: int, seed: int):
    """Return (q, k, v) as contiguous bf16 CPU tensors of shape [B, H, L, d].

    One CPU generator per call, seeded with ``seed``; float32 ``randn`` drawn in
    the order q, k, v and each rounded to bf16 (round to nearest even).
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    out = []
    for _ in range(3):
        x = torch.randn((B, H, L, d), generator=g, dtype=torch.float32)
        out.append(x.to(torch.bfloat16).contiguous())
    return tuple(out)


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
