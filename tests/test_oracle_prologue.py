"""Pins for the prologue oracle (no GPU): "HeyGen x Google Cloud: Bringing Avatar IV
to TPUs", section "Layout as ABI" -- RMSNorm, projection, rotary, head packing.

Each test checks the oracle against something other than itself: complex-number
rotation, closed-form RMS normalisation, scale invariance, rotation invariants,
linearity, and pure-Python brute force on a tiny input.
"""
import math

import numpy as np

import oracle
from sparse_attention_frame_amd import workloads as W


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _angles(S, half, seed):
    return _rand((S, half), seed, 3.0)


def test_rotation_is_complex_multiplication():
    """Pairs (e, e + d/2) as complex numbers a + ib, multiplied by exp(i theta)."""
    B, S, H, d = 2, 7, 3, 16
    u = _rand((B, S, H, d), 1)
    th = _angles(S, d // 2, 2)
    got = oracle.rotate_pairs(u, np.cos(th), np.sin(th))
    z = (u[..., :d // 2] + 1j * u[..., d // 2:]) * np.exp(1j * th)[None, :, None, :]
    np.testing.assert_allclose(got[..., :d // 2], z.real, rtol=0, atol=1e-13)
    np.testing.assert_allclose(got[..., d // 2:], z.imag, rtol=0, atol=1e-13)


def test_rotation_keeps_pair_norms_and_dot_products_depend_on_angle_difference():
    B, S, H, d = 1, 5, 2, 8
    u, v = _rand((B, S, H, d), 3), _rand((B, S, H, d), 4)
    th = _angles(S, d // 2, 5)
    ru = oracle.rotate_pairs(u, np.cos(th), np.sin(th))
    np.testing.assert_allclose(ru[..., :4] ** 2 + ru[..., 4:] ** 2,
                               u[..., :4] ** 2 + u[..., 4:] ** 2, rtol=1e-12, atol=1e-12)
    # the same rotation on q and k leaves q.k unchanged
    rv = oracle.rotate_pairs(v, np.cos(th), np.sin(th))
    np.testing.assert_allclose((ru * rv).sum(-1), (u * v).sum(-1), rtol=1e-12, atol=1e-12)


def test_identity_projection_gives_normalised_rows():
    """W = [I; I; I], no rotation: q = k = v = x / (||x|| / sqrt(C)) * gamma (eps = 0)."""
    B, S, H, d = 1, 6, 2, 8
    C = H * d
    x = _rand((B, S, C), 6)
    gamma = 1 + _rand(C, 7, 0.1)
    w = np.concatenate([np.eye(C)] * 3, axis=0)
    ones, zeros = np.ones((S, d // 2)), np.zeros((S, d // 2))
    q, k, v = oracle.qkv_prologue(x, gamma, w, ones, zeros, H, d, eps=0.0)
    ref = x / (np.linalg.norm(x, axis=-1, keepdims=True) / math.sqrt(C)) * gamma
    for t in (q, k, v):
        np.testing.assert_allclose(t.reshape(B, S, C), ref, rtol=0, atol=1e-13)


def test_scale_invariance_and_linearity():
    B, S, H, d, C = 1, 5, 2, 8, 24
    x = _rand((B, S, C), 8)
    gamma = 1 + _rand(C, 9, 0.1)
    w1, w2 = _rand((3 * H * d, C), 10), _rand((3 * H * d, C), 11)
    th = _angles(S, d // 2, 12)
    c, s = np.cos(th), np.sin(th)
    a = oracle.qkv_prologue(x, gamma, w1, c, s, H, d, eps=0.0)
    b = oracle.qkv_prologue(7.5 * x, gamma, w1, c, s, H, d, eps=0.0)
    for ta, tb in zip(a, b):
        np.testing.assert_allclose(ta, tb, rtol=1e-12, atol=1e-12)
    # every output is linear in W (rotation and packing are linear)
    s12 = oracle.qkv_prologue(x, gamma, w1 + w2, c, s, H, d)
    s1 = oracle.qkv_prologue(x, gamma, w1, c, s, H, d)
    s2 = oracle.qkv_prologue(x, gamma, w2, c, s, H, d)
    for t12, t1, t2 in zip(s12, s1, s2):
        np.testing.assert_allclose(t12, t1 + t2, rtol=1e-12, atol=1e-12)


def test_head_packing_order():
    """Row n of W feeds q, k or v = n // (H*d), head (n // d) % H, element n % d."""
    B, S, H, d, C = 1, 3, 3, 4, 5
    x = _rand((B, S, C), 13)
    w = np.zeros((3 * H * d, C))
    n = 1 * H * d + 2 * d + 3            # k, head 2, element 3
    w[n, 0] = 1.0
    ones, zeros = np.ones((S, d // 2)), np.zeros((S, d // 2))
    q, k, v = oracle.qkv_prologue(x, np.ones(C), w, ones, zeros, H, d, eps=0.0)
    assert not q.any() and not v.any()
    nz = np.argwhere(k != 0)
    assert set(map(tuple, nz[:, 2:])) == {(2, 3)}


def test_brute_force_tiny():
    """Pure-Python loops with math.fsum on the tiny prologue input."""
    pw = W.PRO_TINY
    x, gamma, w, cos, sin = W.make_prologue_inputs_np(pw)
    x = x[:, :40]                         # first 40 tokens keep it quick
    cos, sin = cos[:40], sin[:40]
    H, d, C = pw.heads, pw.head_dim, pw.model_dim
    q, k, v = oracle.qkv_prologue(x, gamma, w, cos, sin, H, d)
    eps = 1e-6
    for s in (0, 17, 39):
        row = [float(t) for t in x[0, s]]
        r = 1.0 / math.sqrt(math.fsum(t * t for t in row) / C + eps)
        xn = [row[c] * r * float(gamma[c]) for c in range(C)]
        y = [math.fsum(xn[c] * float(w[n, c]) for c in range(C)) for n in range(3 * H * d)]
        for which, out in enumerate((q, k, v)):
            for h in range(H):
                base = which * H * d + h * d
                u = y[base:base + d]
                for e in range(d):
                    if which == 2:
                        want = u[e]
                    elif e < d // 2:
                        want = u[e] * float(cos[s, e]) - u[e + d // 2] * float(sin[s, e])
                    else:
                        j = e - d // 2
                        want = u[j] * float(sin[s, j]) + u[e] * float(cos[s, j])
                    assert abs(out[0, s, h, e] - want) <= 1e-12, (which, s, h, e)


def test_rope_tables_are_valid_rotations():
    pw = W.PRO_SMALL
    cos, sin = W.rope_tables(pw)
    assert cos.shape == (pw.seq, pw.head_dim // 2)
    np.testing.assert_allclose(cos.astype(np.float64) ** 2 + sin.astype(np.float64) ** 2, 1.0,
                               rtol=0, atol=1e-6)
    # position 0 (reference frame, row 0, column 0) is the identity
    np.testing.assert_array_equal(cos[0], 1.0)
    np.testing.assert_array_equal(sin[0], 0.0)
