"""Float64 reference for the fused attention prologue (test infrastructure).

Page: "HeyGen x Google Cloud: Bringing Avatar IV to TPUs", section "Layout as
ABI" (Fig. 5): the attention's inputs come from a chain of small operations --
normalisation, rotary embedding, projection, head packing -- which the pages
fuse into one kernel that writes straight into the layout the consumer reads.

Readings (the pages name the steps, not their formulas):
  * normalisation is RMSNorm over the model width C with a weight gamma:
    xn = x / sqrt(mean(x^2) + eps) * gamma;
  * the projection is y = xn W^T with W stored [3*H*d][C] (q, k, v stacked);
  * rotary embedding acts on q and k of every head, on the pairs
    (e, e + d/2), e < d/2, with per-token tables cos[s][e], sin[s][e]:
    (a, b) -> (a cos - b sin, a sin + b cos);
  * head packing writes q, k, v as [B, S, H, d].
All arithmetic is float64 on the given (bf16-representable) inputs.
"""
from __future__ import annotations

import numpy as np


def rms_norm(x, gamma, eps: float = 1e-6):
    """x [B, S, C] -> x / sqrt(mean over C of x^2 + eps) * gamma."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    ms = (x * x).mean(axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rotate_pairs(u, cos, sin):
    """u [B, S, H, d]; cos, sin [S, d/2]: rotate the pairs (e, e + d/2)."""
    u = np.asarray(u, dtype=np.float64)
    half = u.shape[-1] // 2
    c = np.asarray(cos, dtype=np.float64)[None, :, None, :]
    s = np.asarray(sin, dtype=np.float64)[None, :, None, :]
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def qkv_prologue(x, gamma, w, cos, sin, heads: int, head_dim: int, eps: float = 1e-6):
    """RMSNorm -> projection -> rotary (q, k) -> head packing. Returns q, k, v [B, S, H, d]."""
    xn = rms_norm(x, gamma, eps)
    y = xn @ np.asarray(w, dtype=np.float64).T                  # [B, S, 3*H*d]
    B, S, _ = y.shape
    y = y.reshape(B, S, 3, heads, head_dim)
    q, k, v = y[:, :, 0], y[:, :, 1], y[:, :, 2]
    return rotate_pairs(q, cos, sin), rotate_pairs(k, cos, sin), v
