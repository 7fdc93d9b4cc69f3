"""Seeded synthetic workloads shared by the tests, smoke() and bench.py.

This module holds shapes and random-number generation only: none of the
attention or mask arithmetic lives here, so both the GPU path's tests and the
oracle can draw identical inputs from it without sharing any method code.

The shapes stand in for the video models the radial-attention pages evaluate
(HunyuanVideo 5 s 720p, Wan2.1-14B 720p, 4x-longer HunyuanVideo, and a
training step); their latent videos are not available, so Q, K, V (and dO)
are i.i.d. N(0, 1) draws rounded to bf16 (the 1/sqrt(D) that one workload
description mentions is the softmax scale, applied by the kernels).  The work
the kernels do depends only on the shapes and the mask; their speed does
depend on the values, because the clock the GPU sustains depends on the power
the arithmetic draws.
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
    frames: int
    tokens_per_frame: int
    D: int
    T: int
    seed: int
    backward: bool = False
    desc: str = ""
    input_scale: float = 1.0  # Q, K, V are N(0, 1) * input_scale, rounded to bf16

    @property
    def N(self) -> int:
        return self.frames * self.tokens_per_frame

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f8_s256", 1, 2, 8, 256, 64, 64, 1,
                 desc="tiny radial attention fwd: 8 frames x 256 tokens, D=64, 64x64 tiles"),
        Workload("hunyuan_5s_720p", 1, 24, 33, 3600, 128, 128, 2,
                 desc="HunyuanVideo-shaped 5 s 720p fwd: 33 latent frames x 3600 tokens (80x45)"),
        Workload("wan21_720p", 1, 40, 21, 3600, 128, 128, 3,
                 desc="Wan2.1-14B-shaped 720p fwd: 21 latent frames x 3600 tokens"),
        Workload("hunyuan_4x_long", 1, 24, 129, 3600, 128, 128, 4,
                 desc="4x longer HunyuanVideo-shaped fwd: 129 latent frames x 3600 tokens"),
        Workload("train_f66", 1, 24, 66, 3600, 128, 128, 5, backward=True,
                 desc="training step fwd+bwd: 66 latent frames x 3600 tokens"),
    ]
}

ORDER = ["tiny_f8_s256", "hunyuan_5s_720p", "wan21_720p", "hunyuan_4x_long", "train_f66"]


def randn_bf16(shape, gen: torch.Generator, device="cpu", scale: float = 1.0) -> torch.Tensor:
    """i.i.d. N(0,1) drawn in float32, times `scale`, rounded to bf16 (round to
    nearest even)."""
    t = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    if scale != 1.0:
        t = t * scale
    return t.to(torch.bfloat16)


def make_inputs(B: int, H: int, N: int, D: int, seed: int, with_dout: bool = False,
                heads=None, device="cpu", input_scale: float = 1.0):
    """Q, K, V (and dO) as bf16 tensors [B, H, N, D], drawn in that order from
    a ``torch.Generator(device).manual_seed(seed)``.

    ``device="cpu"`` (default) draws with torch's CPU generator; a GPU device
    draws with torch's GPU generator directly in device memory (fast for the
    full-size shapes; a different but equally seeded stream of values).
    ``heads``: optionally keep only these head indices of the full draw (the
    draw itself is always the full [B, H, N, D] so values do not depend on
    which heads are kept).
    ``input_scale`` multiplies the Q, K, V draws (not dO) before rounding.
    """
    g = torch.Generator(device).manual_seed(seed)
    names = ["q", "k", "v"] + (["do"] if with_dout else [])
    out = []
    for name in names:
        t = randn_bf16((B, H, N, D), g, device, input_scale if name != "do" else 1.0)
        if heads is not None:
            t = t[:, list(heads)].contiguous()
        out.append(t)
    return tuple(out)


def workload_inputs(w: Workload, with_dout: bool | None = None, heads=None, device="cpu"):
    wd = w.backward if with_dout is None else with_dout
    return make_inputs(w.B, w.H, w.N, w.D, w.seed, wd, heads, device, w.input_scale)
