"""Float64 reference for frame-aligned window-sparse attention (test infrastructure).

Page: "HeyGen x Google Cloud: Bringing Avatar IV to TPUs".

Token order (section "Hiding collectives" says the mask is defined on one
fixed token order; section "Deleting the mask" says the mask lines up with
frame boundaries): tokens are frame-major, frame 0 is the reference frame,
frames 1..F are the video frames, each of T tokens, so S = (F + 1) * T.

Mask (section "Deleting the mask", Fig. 3): a video-frame query sees the
reference frame and the video frames at most w frames away from its own; the
reference frame's queries see the reference frame only (a reading the pages
leave open; the workload definitions fix it).

All arithmetic is float64. Inputs are the bf16-representable values of the
workload, upcast exactly.
"""
from __future__ import annotations

import numpy as np


def key_frames(query_frame: int, frames: int, window: int) -> list[int]:
    """Frames whose keys a query of ``query_frame`` may attend to (sorted)."""
    if query_frame == 0:
        return [0]
    lo = max(1, query_frame - window)
    hi = min(frames, query_frame + window)
    return [0] + list(range(lo, hi + 1))


def mask_matrix(frames: int, tokens_per_frame: int, window: int) -> np.ndarray:
    """Boolean [S, S] matrix: entry (i, j) is True when query i may see key j."""
    T = tokens_per_frame
    S = (frames + 1) * T
    frame = np.arange(S) // T
    fi = frame[:, None]
    fj = frame[None, :]
    video_pair = (fi >= 1) & (fj >= 1) & (np.abs(fi - fj) <= window)
    return (fj == 0) | video_pair


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax of logits that may hold -inf (each row has a finite entry)."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def _default_scale(d: int, scale) -> float:
    return 1.0 / np.sqrt(d) if scale is None or scale == 0 else float(scale)


def attention_block(qh, kh, vh, frames: int, tokens_per_frame: int, window: int,
                    r0: int, r1: int, scale=None):
    """Rows r0 .. r1-1 of one (batch, head), all inside one query frame: the same
    definition as ``attention`` (dense logits, the mask as -inf, softmax, times v).

    qh, kh, vh: arrays [S, d] of one (batch, head). Returns float64 [r1 - r0, d].
    """
    S, d = kh.shape
    T = tokens_per_frame
    f = r0 // T
    assert (r1 - 1) // T == f, "a block lies inside one query frame"
    sc = _default_scale(d, scale)
    visible = np.isin(np.arange(S) // T, key_frames(f, frames, window))
    s = sc * (np.asarray(qh[r0:r1], dtype=np.float64) @ np.asarray(kh, dtype=np.float64).T)
    s[:, ~visible] = -np.inf
    return _softmax_rows(s) @ np.asarray(vh, dtype=np.float64)


def attention(q, k, v, frames: int, tokens_per_frame: int, window: int, scale=None):
    """O = softmax(scale * q k^T + mask) v for every (batch, head), float64.

    q, k, v: arrays [B, S, H, d]. Returns float64 [B, S, H, d].
    Work is done one query frame at a time to bound memory (T x S logits).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, S, H, d = q.shape
    T = tokens_per_frame
    assert S == (frames + 1) * T
    out = np.empty((B, S, H, d), dtype=np.float64)
    for f in range(frames + 1):
        for b in range(B):
            for h in range(H):
                out[b, f * T:(f + 1) * T, h, :] = attention_block(
                    q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], frames, T, window,
                    f * T, (f + 1) * T, scale)
    return out


def attention_rows(q, k, v, frames: int, tokens_per_frame: int, window: int,
                   b: int, h: int, rows, scale=None):
    """Same definition as ``attention`` for a chosen set of query rows of (b, h).

    Returns float64 [len(rows), d]. Used for sampled parity at full sizes.
    """
    rows = np.asarray(rows, dtype=np.int64)
    d = q.shape[-1]
    S = q.shape[1]
    T = tokens_per_frame
    sc = _default_scale(d, scale)
    kb = np.asarray(k[b, :, h, :], dtype=np.float64)
    vb = np.asarray(v[b, :, h, :], dtype=np.float64)
    qr = np.asarray(q[b, rows, h, :], dtype=np.float64)
    s = sc * (qr @ kb.T)  # [R, S]
    frame_of_key = np.arange(S) // T
    for r, i in enumerate(rows):
        visible = np.isin(frame_of_key, key_frames(int(i) // T, frames, window))
        s[r, ~visible] = -np.inf
    return _softmax_rows(s) @ vb


def head_stats(q, k, scale=None, bound_limit: float = 40.0):
    """Per-(batch, head) quantities of the Cauchy-Schwarz fixed maximum.

    Section "Unchaining softmax" (Fig. 4): every logit is at most the query
    norm times the largest key norm; centring the keys on their mean first
    tightens this and leaves softmax unchanged; a head whose bound is too loose
    (its exponentials would underflow) takes the online path instead.

    mu[b, h]    = mean over all S keys of k               (float64)
    kmax[b, h]  = max over keys of ||k_j - mu||
    qmax[b, h]  = max over queries of ||q_i||
    bound[b, h] = scale * qmax * kmax
    eligible    = bound <= bound_limit   (inclusive; bound_limit < 0 makes every head ineligible)
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d = q.shape[-1]
    sc = _default_scale(d, scale)
    mu = k.mean(axis=1)                                          # [B, H, d]
    kmax = np.sqrt(((k - mu[:, None]) ** 2).sum(axis=-1)).max(axis=1)  # [B, H]
    qmax = np.sqrt((q ** 2).sum(axis=-1)).max(axis=1)            # [B, H]
    bound = sc * qmax * kmax
    eligible = bound <= bound_limit
    return {"mu": mu, "kmax": kmax, "qmax": qmax, "bound": bound, "eligible": eligible}


def row_offsets(q, k, scale=None):
    """Fixed per-row maximum M[b, i, h] = scale * (<q_i, mu> + ||q_i|| * kmax).

    Raw logits minus M equal centred logits minus scale * ||q_i|| * kmax, which
    is <= 0 by Cauchy-Schwarz, for every key of the head and hence for every
    row's visible slice of keys.
    """
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    sc = _default_scale(d, scale)
    st = head_stats(q, k, scale)
    qn = np.sqrt((q ** 2).sum(axis=-1))                       # [B, S, H]
    qmu = np.einsum("bshd,bhd->bsh", q, st["mu"])             # [B, S, H]
    return sc * (qmu + qn * st["kmax"][:, None, :])


def frame_stats(q, k, frames: int, tokens_per_frame: int, window: int, scale=None,
                bound_limit: float = 40.0):
    """Per (batch, head, query frame) tightening of ``head_stats``.

    Section "Unchaining softmax" bounds every logit by the query norm times the
    largest mean-centred key norm. A query row only ever meets the keys of the
    frames it can see (section "Deleting the mask": reference frame plus the
    window), so the largest centred norm over those frames already bounds all
    of its logits. The key mean stays the mean of the whole head: it is one
    shift shared by every row, which softmax ignores.

    mu[b, h]        = mean over all S keys of k                  (as in head_stats)
    kfmax[b, h, f]  = max over the keys of frame f of ||k_j - mu||
    kvis[b, h, g]   = max of kfmax[b, h, f] over the frames f visible from query frame g
    qfmax[b, h, g]  = max over the queries of frame g of ||q_i||
    bound[b, h, g]  = scale * qfmax * kvis
    eligible        = bound <= bound_limit   (per query frame; inclusive;
                                              bound_limit < 0 makes every frame ineligible)
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, S, H, d = q.shape
    T = tokens_per_frame
    assert S == (frames + 1) * T
    sc = _default_scale(d, scale)
    mu = k.mean(axis=1)                                               # [B, H, d]
    knorm = np.sqrt(((k - mu[:, None]) ** 2).sum(axis=-1))           # [B, S, H]
    qnorm = np.sqrt((q ** 2).sum(axis=-1))                           # [B, S, H]
    kfmax = np.empty((B, H, frames + 1))
    qfmax = np.empty((B, H, frames + 1))
    for f in range(frames + 1):
        kfmax[:, :, f] = knorm[:, f * T:(f + 1) * T, :].max(axis=1)
        qfmax[:, :, f] = qnorm[:, f * T:(f + 1) * T, :].max(axis=1)
    kvis = np.empty_like(kfmax)
    for g in range(frames + 1):
        kvis[:, :, g] = kfmax[:, :, key_frames(g, frames, window)].max(axis=-1)
    bound = sc * qfmax * kvis
    eligible = bound <= bound_limit
    return {"mu": mu, "kfmax": kfmax, "kvis": kvis, "qfmax": qfmax, "bound": bound,
            "eligible": eligible}


def frame_row_offsets(q, k, frames: int, tokens_per_frame: int, window: int, scale=None):
    """Fixed per-row maximum with the per-frame bound:
    M[b, i, h] = scale * (<q_i, mu> + ||q_i|| * kvis[b, h, frame(i)]).

    Raw logit minus M = centred logit minus scale * ||q_i|| * kvis, which is
    <= 0 by Cauchy-Schwarz for every key the row can see.
    """
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    T = tokens_per_frame
    sc = _default_scale(d, scale)
    st = frame_stats(q, k, frames, T, window, scale)
    qn = np.sqrt((q ** 2).sum(axis=-1))                       # [B, S, H]
    qmu = np.einsum("bshd,bhd->bsh", q, st["mu"])             # [B, S, H]
    frame = np.arange(q.shape[1]) // T
    kv = np.transpose(st["kvis"], (0, 2, 1))[:, frame, :]     # [B, S, H]
    return sc * (qmu + qn * kv)
