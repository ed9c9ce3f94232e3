"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: hand-written
fixtures, brute force, torch's float64 attention with an independently built
mask, closed forms, exact-value constructions and invariants of the method
("HeyGen x Google Cloud: Bringing Avatar IV to TPUs", sections "Deleting the
mask" and "Unchaining softmax").
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_frame_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_frame_mask(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    return np.array(rows, dtype=bool)


def _token_mask_from_frames(fm, T):
    return np.kron(fm.astype(np.int64), np.ones((T, T), dtype=np.int64)).astype(bool)


def _rand(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape) * scale


# ---------------------------------------------------------------- mask ----

@pytest.mark.parametrize("fname,wl", [("tiny_frame_mask.txt", W.TINY),
                                      ("small_frame_mask.txt", W.SMALL)])
def test_mask_matches_hand_written_fixture(fname, wl):
    fm = _load_frame_mask(fname)
    assert fm.shape == (wl.frames + 1, wl.frames + 1)
    got = oracle.mask_matrix(wl.frames, wl.tokens_per_frame, wl.window)
    np.testing.assert_array_equal(got, _token_mask_from_frames(fm, wl.tokens_per_frame))
    for f in range(wl.frames + 1):
        assert oracle.key_frames(f, wl.frames, wl.window) == list(np.nonzero(fm[f])[0])


def test_frame_pair_counts_golden():
    with open(os.path.join(GOLDEN, "frame_pairs.json")) as f:
        gold = json.load(f)
    for name, g in gold.items():
        if name.startswith("_"):
            continue
        wl = W.ALL[name]
        assert (wl.frames, wl.window) == (g["frames"], g["window"])
        frame_level = oracle.mask_matrix(wl.frames, 1, wl.window)
        assert int(frame_level.sum()) == g["pairs"], name
        # token level at a small T: every visible frame pair contributes T*T pairs
        assert int(oracle.mask_matrix(wl.frames, 3, wl.window).sum()) == 9 * g["pairs"]


# ------------------------------------------------------------ softmax ----

def test_oracle_matches_brute_force_tiny():
    q, k, v = W.make_inputs_np(W.TINY)
    wl = W.TINY
    got = oracle.attention(q, k, v, wl.frames, wl.tokens_per_frame, wl.window)
    ref = np.array(oracle.attention_brute(q.astype(np.float64), k.astype(np.float64),
                                          v.astype(np.float64), wl.frames,
                                          wl.tokens_per_frame, wl.window))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("fname,F,T,w,H,d", [("tiny_frame_mask.txt", 4, 16, 1, 2, 64),
                                             ("small_frame_mask.txt", 8, 16, 2, 3, 128)])
def test_oracle_matches_torch_sdpa_with_fixture_mask(fname, F, T, w, H, d):
    S = (F + 1) * T
    q = _rand((1, S, H, d), 1)
    k = _rand((1, S, H, d), 2) + _rand((1, 1, H, d), 3, 3.0)
    v = _rand((1, S, H, d), 4)
    mask = torch.from_numpy(_token_mask_from_frames(_load_frame_mask(fname), T))
    # torch wants [B, H, S, d]
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).contiguous() for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    ref = ref.permute(0, 2, 1, 3).numpy()
    got = oracle.attention(q, k, v, F, T, w)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_full_window_equals_dense_attention():
    """w >= F-1: video rows see every key, so they equal unmasked attention."""
    F, T, H, d = 5, 16, 2, 64
    S = (F + 1) * T
    q, k, v = _rand((1, S, H, d), 5), _rand((1, S, H, d), 6), _rand((1, S, H, d), 7)
    got = oracle.attention(q, k, v, F, T, F - 1)
    for h in range(H):
        s = (q[0, :, h] @ k[0, :, h].T) / math.sqrt(d)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        dense = (p / p.sum(axis=1, keepdims=True)) @ v[0, :, h]
        np.testing.assert_allclose(got[0, T:, h], dense[T:], rtol=0, atol=1e-12)
        # reference rows: plain attention over the reference frame alone
        s0 = (q[0, :T, h] @ k[0, :T, h].T) / math.sqrt(d)
        p0 = np.exp(s0 - s0.max(axis=1, keepdims=True))
        ref0 = (p0 / p0.sum(axis=1, keepdims=True)) @ v[0, :T, h]
        np.testing.assert_allclose(got[0, :T, h], ref0, rtol=0, atol=1e-12)
    # wider windows change nothing
    np.testing.assert_allclose(oracle.attention(q, k, v, F, T, F + 3), got, rtol=0, atol=0)


def test_zero_query_gives_window_mean():
    F, T, H, d, w = 6, 16, 1, 64, 2
    S = (F + 1) * T
    q = np.zeros((1, S, H, d))
    k, v = _rand((1, S, H, d), 8), _rand((1, S, H, d), 9)
    got = oracle.attention(q, k, v, F, T, w)
    for f in range(F + 1):
        if f == 0:
            frames = [0]
        else:
            frames = [0] + [g for g in range(f - w, f + w + 1) if 1 <= g <= F]
        mean = np.mean(np.concatenate([v[0, g * T:(g + 1) * T, 0] for g in frames]), axis=0)
        np.testing.assert_allclose(got[0, f * T:(f + 1) * T, 0], np.broadcast_to(mean, (T, d)),
                                   rtol=0, atol=1e-13)


def test_constant_value_gives_constant_output():
    F, T, H, d, w = 4, 16, 2, 64, 1
    S = (F + 1) * T
    q, k = _rand((1, S, H, d), 10, 3.0), _rand((1, S, H, d), 11, 3.0)
    v = np.broadcast_to(_rand((1, 1, H, d), 12), (1, S, H, d))
    got = oracle.attention(q, k, v, F, T, w)
    np.testing.assert_allclose(got, np.broadcast_to(v, got.shape), rtol=0, atol=1e-13)


def test_frame_indicator_values_give_zero_mass_outside_window():
    F, T, H, d, w = 6, 16, 2, 64, 1
    S = (F + 1) * T
    q, k = _rand((1, S, H, d), 13), _rand((1, S, H, d), 14)
    v = np.zeros((1, S, H, d))
    for j in range(S):
        v[0, j, :, j // T] = 1.0
    got = oracle.attention(q, k, v, F, T, w)
    for i in range(S):
        f = i // T
        for e in range(F + 1):
            inside = e == 0 or (f >= 1 and 1 <= e <= F and abs(e - f) <= w)
            mass = got[0, i, :, e]
            if inside:
                assert np.all(mass > 0)
            else:
                assert np.all(mass == 0.0)
        np.testing.assert_allclose(got[0, i, :, :F + 1].sum(axis=-1), 1.0, rtol=0, atol=1e-14)


def test_permutation_inside_a_frame_is_invisible():
    F, T, H, d, w = 4, 16, 2, 64, 1
    S = (F + 1) * T
    q, k, v = _rand((1, S, H, d), 15), _rand((1, S, H, d), 16), _rand((1, S, H, d), 17)
    perm = np.arange(S)
    g = np.random.default_rng(18)
    for f in range(F + 1):
        perm[f * T:(f + 1) * T] = f * T + g.permutation(T)
    a = oracle.attention(q, k, v, F, T, w)
    b = oracle.attention(q, k[:, perm], v[:, perm], F, T, w)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_key_centring_leaves_output_unchanged():
    """Section "Unchaining softmax": subtracting the key mean is softmax-invariant."""
    wl = W.TINY
    q, k, v = W.make_inputs_np(wl)
    mu = k.astype(np.float64).mean(axis=1, keepdims=True)
    a = oracle.attention(q, k, v, wl.frames, wl.tokens_per_frame, wl.window)
    b = oracle.attention(q, k.astype(np.float64) - mu, v, wl.frames, wl.tokens_per_frame,
                         wl.window)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_attention_rows_matches_full():
    wl = W.SMALL
    q, k, v = W.make_inputs_np(wl)
    full = oracle.attention(q, k, v, wl.frames, wl.tokens_per_frame, wl.window)
    rows = [0, 207, 208, 415, 1000, 1871]
    for h in (0, 5):
        got = oracle.attention_rows(q, k, v, wl.frames, wl.tokens_per_frame, wl.window, 0, h,
                                    rows)
        np.testing.assert_allclose(got, full[0, rows, h], rtol=0, atol=1e-13)


# -------------------------------------------------------------- bound ----

def _closed_form_heads(a_values, qbig=16.0):
    """d = 64, S = 128: k_j = c + a * (+-e_{j mod 64}) so mu = c and kmax = a exactly;
    q_i = 2 * e_0 except row 5 with q_5 = qbig * e_0, so qmax = qbig."""
    d, S = 64, 128
    H = len(a_values)
    c = np.arange(1, d + 1, dtype=np.float64) / 8.0
    k = np.empty((1, S, H, d))
    q = np.zeros((1, S, H, d))
    for h, a in enumerate(a_values):
        for j in range(S):
            k[0, j, h] = c
            k[0, j, h, j % d] += a if j < d else -a
        q[0, :, h, 0] = 2.0
        q[0, 5, h, 0] = qbig
    return q, k


def test_bound_closed_form_and_inclusive_threshold():
    # scale = 1/8 (d = 64): bound = qmax * kmax / 8 = 16 * a / 8 = 2a
    q, k = _closed_form_heads([20.0, 20.5, 3.0])
    st = oracle.head_stats(q, k)
    for h in range(3):
        np.testing.assert_allclose(st["mu"][0, h], np.arange(1, 65) / 8.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(st["kmax"][0], [20.0, 20.5, 3.0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(st["qmax"][0], [16.0, 16.0, 16.0], rtol=0, atol=0)
    np.testing.assert_allclose(st["bound"][0], [40.0, 41.0, 6.0], rtol=0, atol=1e-12)
    assert list(st["eligible"][0]) == [True, False, True]       # 40 is still eligible
    st_forced = oracle.head_stats(q, k, bound_limit=-1.0)
    assert not st_forced["eligible"].any()


def test_row_offset_is_tight_when_query_aligns_with_widest_key():
    """q_i parallel to k_0 - mu (key 0 is in the reference frame, visible to every row):
    the fixed maximum equals that row's true maximum logit exactly."""
    q, k = _closed_form_heads([20.0])
    M = oracle.row_offsets(q, k)                            # [1, S, 1]
    s = (q[0, :, 0] @ k[0, :, 0].T) / 8.0                   # every key visible (F=1, T=64, w=1)
    np.testing.assert_allclose(M[0, :, 0], s.max(axis=1), rtol=0, atol=1e-12)
    np.testing.assert_allclose(M[0, :, 0], s[:, 0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_fixed_max_bounds_every_visible_logit(name):
    wl = W.ALL[name]
    q, k, v = W.make_inputs_np(wl)
    M = oracle.row_offsets(q, k)
    mask = oracle.mask_matrix(wl.frames, wl.tokens_per_frame, wl.window)
    sc = 1.0 / math.sqrt(wl.head_dim)
    for h in range(wl.heads):
        s = sc * (q[0, :, h].astype(np.float64) @ k[0, :, h].astype(np.float64).T)
        smax = np.where(mask, s, -np.inf).max(axis=1)
        gap = M[0, :, h] - smax
        assert gap.min() >= -1e-9
        # and the bound keeps every exponent above exp(-2 * bound)
        bound = oracle.head_stats(q, k)["bound"][0, h]
        smin = np.where(mask, s, np.inf).min(axis=1)
        assert np.all(M[0, :, h] - smin <= 2 * bound + 1e-9)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["720p", "stress"])
def test_fixed_max_bounds_sampled_rows_full_size(name):
    wl = W.ALL[name]
    q, k, v = W.make_inputs_np(wl)
    M = oracle.row_offsets(q, k)
    sc = 1.0 / math.sqrt(wl.head_dim)
    T = wl.tokens_per_frame
    g = np.random.default_rng(7)
    rows = np.concatenate([[0, T - 1, T, 2 * T - 1, wl.seq - 1], g.integers(0, wl.seq, 64)])
    for h in range(wl.heads):
        s = sc * (q[0, rows, h].astype(np.float64) @ k[0, :, h].astype(np.float64).T)
        for r, i in enumerate(rows):
            vis = np.isin(np.arange(wl.seq) // T, oracle.key_frames(int(i) // T, wl.frames,
                                                                    wl.window))
            assert M[0, i, h] - s[r, vis].max() >= -1e-9


@pytest.mark.slow
def test_seeded_workload_eligibility_matches_definitions():
    """Tiny and 720p: every head eligible; stress: exactly heads 3, 7, 11, 15 are not."""
    for name, expect_bad in (("tiny", ()), ("720p", ()), ("stress", (3, 7, 11, 15))):
        wl = W.ALL[name]
        q, k, _ = W.make_inputs_np(wl)
        st = oracle.head_stats(q, k)
        bad = tuple(int(h) for h in np.nonzero(~st["eligible"][0])[0])
        assert bad == expect_bad, (name, st["bound"])
        # keep far from the knife edge so the fp32 comparison on the GPU agrees
        assert np.all(np.abs(st["bound"] - 40.0) > 1.0)


# ------------------------------------------------------- frame bound ----

def _closed_form_frames(a=(1.0, 2.0, 7.0, 3.0, 5.0)):
    """F = 4, T = 16, d = 64, w = 1, one head. Frame f holds c + a_f*e_t (local t < 8) and
    c - a_f*e_{t-8} (t >= 8): every frame's keys average to c, so mu = c and every centred
    key of frame f has norm a_f exactly. Queries are 2*e_0 except local row 3 of frame g,
    which is qg*e_0."""
    F, T, d = 4, 16, 64
    qg = [16.0, 8.0, 48.0, 40.0, 64.0]
    c = np.arange(1, d + 1, dtype=np.float64) / 8.0
    S = (F + 1) * T
    k = np.empty((1, S, 1, d))
    q = np.zeros((1, S, 1, d))
    for f in range(F + 1):
        for t in range(T):
            j = f * T + t
            k[0, j, 0] = c
            if t < 8:
                k[0, j, 0, t] += a[f]
            else:
                k[0, j, 0, t - 8] -= a[f]
            q[0, j, 0, 0] = 2.0
        q[0, f * T + 3, 0, 0] = qg[f]
    return q, k, F, T, 1


def test_frame_bound_closed_form_and_inclusive_threshold():
    q, k, F, T, w = _closed_form_frames()
    st = oracle.frame_stats(q, k, F, T, w)
    np.testing.assert_allclose(st["mu"][0, 0], np.arange(1, 65) / 8.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(st["kfmax"][0, 0], [1, 2, 7, 3, 5], rtol=0, atol=1e-13)
    # visible frames: 0 -> {0}; 1 -> {0,1,2}; 2 -> {0,1,2,3}; 3 -> {0,2,3,4}; 4 -> {0,3,4}
    np.testing.assert_allclose(st["kvis"][0, 0], [1, 7, 7, 7, 5], rtol=0, atol=1e-13)
    np.testing.assert_allclose(st["qfmax"][0, 0], [16, 8, 48, 40, 64], rtol=0, atol=0)
    # scale 1/8: bounds 2, 7, 42, 35, 40 -- 40 is still eligible
    np.testing.assert_allclose(st["bound"][0, 0], [2, 7, 42, 35, 40], rtol=0, atol=1e-12)
    assert list(st["eligible"][0, 0]) == [True, True, False, True, True]
    # the per-head bound of the same inputs is 64 * 7 / 8 = 56: the whole head would fail
    hs = oracle.head_stats(q, k)
    np.testing.assert_allclose(hs["bound"][0, 0], 56.0, rtol=0, atol=1e-12)
    assert not oracle.frame_stats(q, k, F, T, w, bound_limit=-1.0)["eligible"].any()


def test_frame_bound_counts_the_reference_frame():
    """Reference frame widest except for frame 2: frame 4 (sees 0, 3, 4) takes its bound from
    the reference frame's keys, frames 1..3 from frame 2's."""
    q, k, F, T, w = _closed_form_frames(a=(6.0, 2.0, 7.0, 3.0, 5.0))
    st = oracle.frame_stats(q, k, F, T, w)
    np.testing.assert_allclose(st["kvis"][0, 0], [6, 7, 7, 7, 6], rtol=0, atol=1e-13)
    np.testing.assert_allclose(st["bound"][0, 0], [12, 7, 42, 35, 48], rtol=0, atol=1e-12)
    assert list(st["eligible"][0, 0]) == [True, True, False, True, False]


def test_frame_row_offset_is_tight_on_the_widest_visible_key():
    """Row 3 of frames 1 and 4 points along e_0, the direction of the widest key they can
    see (frame 2's key 0 with norm 7, frame 4's key 0 with norm 5): M equals the row's true
    maximum logit there."""
    q, k, F, T, w = _closed_form_frames()
    M = oracle.frame_row_offsets(q, k, F, T, w)
    mask = oracle.mask_matrix(F, T, w)
    s = (q[0, :, 0] @ k[0, :, 0].T) / 8.0
    smax = np.where(mask, s, -np.inf).max(axis=1)
    assert np.all(M[0, :, 0] - smax >= -1e-12)
    for g in (1, 4):
        i = g * T + 3
        np.testing.assert_allclose(M[0, i, 0], smax[i], rtol=0, atol=1e-12)


def test_frame_bound_matches_brute_force_tiny():
    """Visible key sets enumerated as in the brute-force module, norms with math.fsum."""
    from oracle.brute import visible_keys

    wl = W.TINY
    q, k, _ = W.make_inputs_np(wl)
    F, T, w, d = wl.frames, wl.tokens_per_frame, wl.window, wl.head_dim
    st = oracle.frame_stats(q, k, F, T, w)
    sc = 1.0 / math.sqrt(d)
    for h in range(wl.heads):
        mu = [math.fsum(float(k[0, j, h, t]) for j in range(wl.seq)) / wl.seq for t in range(d)]
        for g in range(F + 1):
            keys = visible_keys(g * T, F, T, w)
            kv = max(math.sqrt(math.fsum((float(k[0, j, h, t]) - mu[t]) ** 2 for t in range(d)))
                     for j in keys)
            qf = max(math.sqrt(math.fsum(float(q[0, i, h, t]) ** 2 for t in range(d)))
                     for i in range(g * T, (g + 1) * T))
            assert abs(st["kvis"][0, h, g] - kv) <= 1e-12
            assert abs(st["qfmax"][0, h, g] - qf) <= 1e-12
            assert abs(st["bound"][0, h, g] - sc * qf * kv) <= 1e-12


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_frame_bound_is_tighter_and_still_bounds_every_visible_logit(name):
    wl = W.ALL[name]
    q, k, _ = W.make_inputs_np(wl)
    F, T, w = wl.frames, wl.tokens_per_frame, wl.window
    fs = oracle.frame_stats(q, k, F, T, w)
    hs = oracle.head_stats(q, k)
    # a max over a subset, and every frame is visible from some query frame
    assert np.all(fs["kvis"] <= hs["kmax"][..., None])
    np.testing.assert_array_equal(fs["kvis"].max(axis=-1), hs["kmax"])
    np.testing.assert_array_equal(fs["kfmax"].max(axis=-1), hs["kmax"])
    np.testing.assert_array_equal(fs["qfmax"].max(axis=-1), hs["qmax"])
    assert np.all(fs["bound"] <= hs["bound"][..., None] + 1e-12)
    Mf = oracle.frame_row_offsets(q, k, F, T, w)
    Mh = oracle.row_offsets(q, k)
    assert np.all(Mf <= Mh + 1e-9)
    mask = oracle.mask_matrix(F, T, w)
    sc = 1.0 / math.sqrt(wl.head_dim)
    frame = np.arange(wl.seq) // T
    for h in range(wl.heads):
        s = sc * (q[0, :, h].astype(np.float64) @ k[0, :, h].astype(np.float64).T)
        smax = np.where(mask, s, -np.inf).max(axis=1)
        smin = np.where(mask, s, np.inf).min(axis=1)
        assert (Mf[0, :, h] - smax).min() >= -1e-9
        assert np.all(Mf[0, :, h] - smin <= 2 * fs["bound"][0, h, frame] + 1e-9)


def test_frame_bound_full_window_reduces_to_head_bound():
    """w >= F: every video frame sees every frame, so its kvis is the head's kmax."""
    wl = W.TINY
    q, k, _ = W.make_inputs_np(wl)
    fs = oracle.frame_stats(q, k, wl.frames, wl.tokens_per_frame, wl.frames)
    hs = oracle.head_stats(q, k)
    np.testing.assert_array_equal(fs["kvis"][:, :, 1:],
                                  np.broadcast_to(hs["kmax"][..., None], fs["kvis"][:, :, 1:].shape))
    np.testing.assert_array_equal(fs["kvis"][:, :, 0], fs["kfmax"][:, :, 0])
