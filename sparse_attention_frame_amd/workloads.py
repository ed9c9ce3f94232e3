"""Seeded synthetic inputs for frame-aligned window-sparse attention.

This module only draws random tensors; it contains none of the attention
arithmetic. Both the HIP path (through the tests and the bench) and the CPU
oracle consume exactly the tensors produced here.

The shapes model the self-attention of the super-resolution transformer in
the Avatar IV pipeline ("HeyGen x Google Cloud: Bringing Avatar IV to TPUs",
section "Deleting the mask"): one reference frame followed by F latent video
frames of T tokens each, laid out frame-major, heads independent. Real
activations are not available, so q and v are standard normal and every key of
a head carries a shared random offset ``c``, modelling the sizeable component
that keys have in common according to the section "Unchaining softmax". Values are drawn in fp32
and rounded to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    frames: int            # F: latent video frames (the reference frame is extra)
    tokens_per_frame: int  # T
    heads: int             # H
    head_dim: int          # d
    window: int            # w: a video frame sees video frames within +-w
    sigma_c: float         # std-dev of the per-head shared key component
    seed: int
    batch: int = 1
    boost_heads: Tuple[int, ...] = field(default_factory=tuple)  # q and k scaled by boost
    boost: float = 6.0
    boost_key_frames: Tuple[int, ...] = field(default_factory=tuple)  # k of these frames scaled

    @property
    def seq(self) -> int:
        return (self.frames + 1) * self.tokens_per_frame

    def with_window(self, w: int, name: str | None = None) -> "Workload":
        return replace(self, window=w, name=name or f"{self.name}_w{w}")


TINY = Workload("tiny", frames=4, tokens_per_frame=48, heads=2, head_dim=64,
                window=1, sigma_c=2.0, seed=1000)
SMALL = Workload("small", frames=8, tokens_per_frame=208, heads=8, head_dim=128,
                 window=2, sigma_c=3.0, seed=1001)
P720 = Workload("720p", frames=13, tokens_per_frame=3600, heads=12, head_dim=128,
                window=2, sigma_c=3.0, seed=1002)
P1080 = Workload("1080p", frames=5, tokens_per_frame=8160, heads=12, head_dim=128,
                 window=1, sigma_c=3.0, seed=1003)
STRESS = Workload("stress", frames=13, tokens_per_frame=3600, heads=16, head_dim=128,
                  window=2, sigma_c=3.0, seed=1004, boost_heads=(3, 7, 11, 15))
STRESS_FULL = STRESS.with_window(13, "stress_w13")
# 720p geometry whose last video frame carries keys 6x wider than the rest (all heads): the
# per-head bound is then loose everywhere, the per-visible-frame bound only near that frame.
OUTLIER = Workload("outlier", frames=13, tokens_per_frame=3600, heads=12, head_dim=128,
                   window=2, sigma_c=3.0, seed=1005, boost_key_frames=(13,))

ALL = {w.name: w for w in (TINY, SMALL, P720, P1080, STRESS, STRESS_FULL)}


def make_inputs_np(wl: Workload):
    """q, k, v as float32 numpy arrays [B, S, H, d] holding bf16-representable values."""
    import torch

    rng = np.random.default_rng(wl.seed)
    shape = (wl.batch, wl.seq, wl.heads, wl.head_dim)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    c = rng.standard_normal((wl.batch, wl.heads, wl.head_dim), dtype=np.float32)
    c *= np.float32(wl.sigma_c)
    k += c[:, None, :, :]
    for h in wl.boost_heads:
        q[:, :, h, :] *= np.float32(wl.boost)
        k[:, :, h, :] *= np.float32(wl.boost)
    T = wl.tokens_per_frame
    for f in wl.boost_key_frames:
        k[:, f * T:(f + 1) * T, :, :] *= np.float32(wl.boost)
    out = []
    for x in (q, k, v):
        # torch's float32 -> bfloat16 cast rounds to nearest even
        out.append(torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy())
    return tuple(out)


def make_inputs(wl: Workload):
    """q, k, v as contiguous torch.bfloat16 CPU tensors [B, S, H, d]."""
    import torch

    return tuple(torch.from_numpy(x).to(torch.bfloat16) for x in make_inputs_np(wl))


# ---- inputs of the fused attention prologue (RMSNorm -> projection -> rotary -> packing) ----

@dataclass(frozen=True)
class PrologueWorkload:
    name: str
    frames: int            # F video frames (+ the reference frame)
    grid_h: int            # latent patch grid of one frame: T = grid_h * grid_w tokens
    grid_w: int
    heads: int
    head_dim: int
    model_dim: int         # C, the width of the hidden states
    seed: int
    batch: int = 1

    @property
    def tokens_per_frame(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def seq(self) -> int:
        return (self.frames + 1) * self.tokens_per_frame


PRO_TINY = PrologueWorkload("pro_tiny", frames=4, grid_h=6, grid_w=8, heads=4, head_dim=64,
                            model_dim=256, seed=2000)
PRO_SMALL = PrologueWorkload("pro_small", frames=8, grid_h=13, grid_w=16, heads=8, head_dim=128,
                             model_dim=1024, seed=2001)
PRO_720P = PrologueWorkload("pro_720p", frames=13, grid_h=45, grid_w=80, heads=12, head_dim=128,
                            model_dim=1536, seed=2002)
PROLOGUE = {w.name: w for w in (PRO_TINY, PRO_SMALL, PRO_720P)}


def rope_tables(pw: PrologueWorkload, base: float = 10000.0):
    """cos, sin [S, d/2] float32 for 3-axis positions (frame, row, column) of every token:
    the d/2 rotation pairs are split over the three axes (a quarter each for the frame
    axis, the rest halved between rows and columns), frequencies base^(-i/n) per axis.
    The reference frame has frame position 0, video frame f position f."""
    half = pw.head_dim // 2
    nt = half // 4
    nh = (half - nt) // 2
    nw = half - nt - nh
    T = pw.tokens_per_frame
    tok = np.arange(pw.seq)
    pos = np.stack([tok // T, (tok % T) // pw.grid_w, tok % pw.grid_w], axis=1).astype(np.float64)
    ang = []
    for axis, n in enumerate((nt, nh, nw)):
        freq = base ** (-np.arange(n) / n)
        ang.append(pos[:, axis:axis + 1] * freq[None, :])
    ang = np.concatenate(ang, axis=1)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def make_prologue_inputs_np(pw: PrologueWorkload):
    """x [B, S, C], gamma [C], w [3*H*d, C] (bf16-representable float32) and the rope tables."""
    import torch

    rng = np.random.default_rng(pw.seed)
    C, N = pw.model_dim, 3 * pw.heads * pw.head_dim
    x = rng.standard_normal((pw.batch, pw.seq, C), dtype=np.float32)
    gamma = (1.0 + 0.1 * rng.standard_normal(C)).astype(np.float32)
    w = (rng.standard_normal((N, C)) / np.sqrt(C)).astype(np.float32)
    out = [torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy() for a in (x, gamma, w)]
    cos, sin = rope_tables(pw)
    return (*out, cos, sin)
