"""Pure-Python brute force for tiny inputs (test infrastructure).

Page: "HeyGen x Google Cloud: Bringing Avatar IV to TPUs", section "Deleting
the mask" (Fig. 3). Independent of ``attention.py``: the visible keys of a
query are built by listing the reference frame's tokens and then the tokens
of each video frame inside the window, never from a mask formula; the
softmax is written out with an explicit maximum and ``math.fsum``.
"""
from __future__ import annotations

import math


def visible_keys(i: int, frames: int, T: int, window: int) -> list[int]:
    keys = list(range(0, T))               # reference frame: always visible
    f = i // T
    if f >= 1:
        for g in range(f - window, f + window + 1):
            if 1 <= g <= frames:
                keys.extend(range(g * T, (g + 1) * T))
    return keys


def attention_brute(q, k, v, frames: int, T: int, window: int, scale=None):
    """q, k, v: nested sequences or arrays [B][S][H][d]. Returns a nested list."""
    B = len(q)
    S = len(q[0])
    H = len(q[0][0])
    d = len(q[0][0][0])
    sc = 1.0 / math.sqrt(d) if not scale else float(scale)
    out = [[[[0.0] * d for _ in range(H)] for _ in range(S)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(S):
                keys = visible_keys(i, frames, T, window)
                qi = [float(x) for x in q[b][i][h]]
                logits = []
                for j in keys:
                    kj = k[b][j][h]
                    logits.append(sc * math.fsum(qi[t] * float(kj[t]) for t in range(d)))
                m = max(logits)
                w = [math.exp(s - m) for s in logits]
                z = math.fsum(w)
                for t in range(d):
                    out[b][i][h][t] = math.fsum(w[n] * float(v[b][j][h][t])
                                                for n, j in enumerate(keys)) / z
    return out
