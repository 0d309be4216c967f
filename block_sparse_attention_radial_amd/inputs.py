"""Seeded synthetic workloads for the radial attention forward pass.

This module only describes workload shapes and draws the random Q/K/V tensors. It holds
none of the method's arithmetic (no mask rule, no softmax), so both the CPU oracle side
and the HIP side of a test can take their inputs from it without sharing method code.

Shapes follow the video token grids the method is evaluated on: frames x tokens-per-frame
for Wan2.1-14B and HunyuanVideo, plus a 4x longer Wan-shaped video ("Radial Attention:
O(n log n) Sparse Attention with Energy Decay for Long Video Generation", paper summary,
Outline: up to 4x longer videos). Real activations are not available; Q, K and V are
N(0, sigma^2) draws, rounded to bf16 (round-to-nearest-even) before either side sees them.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    """One attention problem: batch, heads, head_dim and the video token grid."""

    name: str
    batch: int
    heads: int
    head_dim: int
    frames: int
    tokens_per_frame: int
    w0: int
    sigma: float
    block: int = 128
    grid_w: int | None = None  # frames as grids of this width (2-D distance); None: 1-D

    @property
    def n(self) -> int:
        """Sequence length: frames x tokens per frame, frame-major."""
        return self.frames * self.tokens_per_frame

    @property
    def scale(self) -> float:
        """Softmax scale head_dim**-0.5."""
        return float(self.head_dim) ** -0.5

    @property
    def nb(self) -> int:
        return (self.n + self.block - 1) // self.block


WORKLOADS: dict[str, Workload] = {
    # 4 frames x 256 tokens, W0 = 256: small enough for the oracle in seconds.
    "tiny": Workload("tiny", 1, 1, 64, 4, 256, 256, 1.0),
    # 8 frames x 1024 tokens, W0 = 512, inputs scaled by 0.5.
    "small": Workload("small", 1, 8, 64, 8, 1024, 512, 0.5),
    # Wan2.1-14B token grid: 21 latent frames x 1560 tokens, 40 heads of 128.
    "wan": Workload("wan2.1-14b-shaped", 1, 40, 128, 21, 1560, 1560, 1.0),
    # HunyuanVideo token grid: 33 latent frames x 3600 tokens, 24 heads of 128.
    "hunyuan": Workload("hunyuanvideo-shaped", 1, 24, 128, 33, 3600, 3600, 1.0),
    # Wan-shaped heads with a 4x longer video: 84 frames x 1560 tokens.
    "long4x": Workload("4x-long-wan-shaped", 1, 40, 128, 84, 1560, 1560, 1.0),
    # The same token grids with the 2-D grid distance: Wan's 1560 tokens per frame as
    # 30 rows of 52, HunyuanVideo's 3600 as 45 rows of 80. W0 = rows + columns - 1 is the
    # smallest window that keeps a frame dense at frame distance 0 (the 1-D workloads'
    # W0 = S does the same for the 1-D distance).
    "wan-grid": Workload("wan2.1-14b-shaped-grid", 1, 40, 128, 21, 1560, 81, 1.0, grid_w=52),
    "hunyuan-grid": Workload("hunyuanvideo-shaped-grid", 1, 24, 128, 33, 3600, 124, 1.0,
                             grid_w=80),
}


def draw_qkv_f32(wl: Workload, seed: int = 0, device: str | torch.device = "cpu",
                 heads: range | None = None):
    """Draw q, k, v (in that order) as fp32 N(0, sigma^2) tensors of shape [B, H, n, D].

    One generator on `device`, seeded with `seed`. `heads` restricts the draw to a
    sub-range of heads: the generator still advances through every head in order,
    so a head's values do not depend on which heads are requested.
    """
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    hs = range(wl.heads) if heads is None else heads
    out = []
    for _ in range(3):
        parts = []
        for b in range(wl.batch):
            for h in range(wl.heads):
                x = torch.randn((wl.n, wl.head_dim), generator=g, dtype=torch.float32,
                                device=device)
                if h in hs:
                    parts.append(x)
        t = torch.stack(parts).reshape(wl.batch, len(hs), wl.n, wl.head_dim)
        out.append(t * wl.sigma)
    return tuple(out)


def draw_qkv(wl: Workload, seed: int = 0, device: str | torch.device = "cpu",
             heads: range | None = None):
    """The same draws as `draw_qkv_f32`, rounded to bf16 (round-to-nearest-even)."""
    return tuple(x.to(torch.bfloat16) for x in draw_qkv_f32(wl, seed, device, heads))


def draw_packed_qkv(total: int, heads: int, head_dim: int, sigma: float = 1.0, seed: int = 0,
                    device: str | torch.device = "cpu"):
    """Packed (varlen) q, k, v of shape [total_tokens, H, D]: N(0, sigma^2) fp32 draws from
    one generator seeded with `seed`, in the order q, k, v, rounded to bf16."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return tuple((torch.randn((total, heads, head_dim), generator=g, dtype=torch.float32,
                              device=device) * sigma).to(torch.bfloat16) for _ in range(3))
