"""GPU parity of the per-visible-frame bound (plan option bound_mode = 1).

Section "Unchaining softmax" of "HeyGen x Google Cloud: Bringing Avatar IV to
TPUs" bounds a row's logits by its query norm times the largest mean-centred
key norm; with bound_mode 1 the largest norm is taken over the frames the
row's query frame can see (section "Deleting the mask"), and eligibility is
decided per (batch, head, query frame). The oracle's ``frame_stats`` defines
the expected norms, bounds and flags; the output must meet the same tolerance
as the per-head mode, and the flags must match exactly.
"""
import sys

import numpy as np
import pytest

import oracle
from sparse_attention_frame_amd import workloads as W

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
REL_L2 = 5e-3


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def sfa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import sparse_attention_frame_amd as m

    m.lib()
    return m


def to_dev(*xs):
    return [torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda() for x in xs]


def assert_close(got, ref, what):
    d = np.asarray(got, np.float64) - np.asarray(ref, np.float64)
    mx = float(np.abs(d).max())
    rl = float(np.linalg.norm(d) / np.linalg.norm(ref))
    say(f"  {what}: max_abs={mx:.3e} rel_l2={rl:.3e}")
    assert mx <= MAX_ABS and rl <= REL_L2, (what, mx, rl)


def geom(wl):
    return (wl.batch, wl.heads, wl.head_dim, wl.frames, wl.tokens_per_frame, wl.window)


def check_frame_stats(sfa, plan, ws, wl, q_np, k_np, mode, limit=40.0):
    got = sfa.frame_stats(plan, ws)
    if mode == 1:
        ref = oracle.frame_stats(q_np, k_np, wl.frames, wl.tokens_per_frame, wl.window,
                                 bound_limit=limit)
        kvis, bound, elig = ref["kvis"], ref["bound"], ref["eligible"]
    else:
        hs = oracle.head_stats(q_np, k_np, bound_limit=limit)
        shape = got["kvis"].shape
        kvis = np.broadcast_to(hs["kmax"][..., None], shape)
        bound = np.broadcast_to(hs["bound"][..., None], shape)
        elig = np.broadcast_to(hs["eligible"][..., None], shape)
    np.testing.assert_array_equal(got["eligible"], elig)
    np.testing.assert_allclose(got["kvis"], kvis, rtol=1e-4)
    np.testing.assert_allclose(got["bound"], bound, rtol=1e-4)
    # the head flag is set exactly when every query frame of the head is eligible
    np.testing.assert_array_equal(sfa.head_stats(plan, ws)["eligible"], elig.all(axis=-1))
    return got


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_frame_bound_full_parity(sfa, name):
    wl = W.ALL[name]
    say(f"[frame_bound_full] {name}")
    q_np, k_np, v_np = W.make_inputs_np(wl)
    q, k, v = to_dev(q_np, k_np, v_np)
    plan = sfa.Plan(*geom(wl), bound_mode=1)
    assert plan.info["bound_mode"] == 1
    out, ws = sfa.attention(plan, q, k, v)
    torch.cuda.synchronize()
    st = check_frame_stats(sfa, plan, ws, wl, q_np, k_np, 1)
    assert st["eligible"].all()
    ref = oracle.attention(q_np, k_np, v_np, wl.frames, wl.tokens_per_frame, wl.window)
    assert_close(out.float().cpu().numpy(), ref, f"{name} frame bound")


SMALL_OUTLIER = W.Workload("small_outlier", frames=6, tokens_per_frame=48, heads=2,
                           head_dim=128, window=1, sigma_c=3.0, seed=1006,
                           boost_key_frames=(6,))


@pytest.mark.parametrize("mode", [0, 1])
def test_outlier_frame_mixes_paths_inside_a_head(sfa, mode):
    """One frame with 6x wider keys: per head every frame is ineligible; per visible frame
    only the query frames that see it are, so one head runs both paths."""
    wl = SMALL_OUTLIER
    say(f"[outlier_small] mode {mode}")
    q_np, k_np, v_np = W.make_inputs_np(wl)
    q, k, v = to_dev(q_np, k_np, v_np)
    plan = sfa.Plan(*geom(wl), bound_mode=mode)
    out, ws = sfa.attention(plan, q, k, v)
    torch.cuda.synchronize()
    st = check_frame_stats(sfa, plan, ws, wl, q_np, k_np, mode)
    if mode == 0:
        assert not st["eligible"].any()
    else:
        # frames 5 and 6 see frame 6; frames 0..4 do not
        assert not st["eligible"][:, :, 5:].any() and st["eligible"][:, :, :5].all()
    ref = oracle.attention(q_np, k_np, v_np, wl.frames, wl.tokens_per_frame, wl.window)
    assert_close(out.float().cpu().numpy(), ref, f"small outlier mode {mode}")


def test_outlier_full_size_sampled(sfa):
    """720p geometry, last frame's keys 6x wider, the benchmark's launch configuration."""
    wl = W.OUTLIER
    say("[outlier_720p] generating inputs")
    q_np, k_np, v_np = W.make_inputs_np(wl)
    q, k, v = to_dev(q_np, k_np, v_np)
    T = wl.tokens_per_frame
    rows = set()
    for f in range(wl.frames + 1):
        rows.update({f * T, f * T + 17, f * T + T // 2, (f + 1) * T - 1})
    rows = np.array(sorted(rows))
    ridx = torch.from_numpy(rows).cuda()
    for mode in (1, 0):
        say(f"[outlier_720p] mode {mode}")
        plan = sfa.Plan(*geom(wl), bound_mode=mode)
        out, ws = sfa.attention(plan, q, k, v)
        torch.cuda.synchronize()
        st = check_frame_stats(sfa, plan, ws, wl, q_np, k_np, mode)
        if mode == 1:
            assert st["eligible"][:, :, :11].all() and not st["eligible"][:, :, 11:].any()
        else:
            assert not st["eligible"].any()
        got = out[0, ridx].float().cpu().numpy()
        heads = range(wl.heads) if mode == 1 else (0, 7)
        for h in heads:
            ref = oracle.attention_rows(q_np, k_np, v_np, wl.frames, T, wl.window, 0, h, rows)
            assert_close(got[:, h], ref, f"outlier mode {mode} head {h}")


@pytest.mark.parametrize("F,T,w,H,d,B", [(0, 16, 0, 1, 64, 1), (3, 80, 5, 3, 128, 1),
                                         (5, 32, 2, 1, 64, 1), (4, 112, 1, 2, 128, 2)])
@pytest.mark.parametrize("limit", [40.0, -1.0])
def test_frame_bound_ragged(sfa, F, T, w, H, d, B, limit):
    say(f"[frame_bound_ragged] F={F} T={T} w={w} H={H} d={d} B={B} limit={limit}")
    S = (F + 1) * T
    g = np.random.default_rng(F * 1000 + T + w + 7)
    q_np = g.standard_normal((B, S, H, d)).astype(np.float32)
    k_np = (g.standard_normal((B, S, H, d)) + 3 * g.standard_normal((B, 1, H, d))).astype(
        np.float32)
    k_np[:, F * T:] *= 6.0                    # the last frame's keys are outliers
    v_np = g.standard_normal((B, S, H, d)).astype(np.float32)
    q, k, v = to_dev(q_np, k_np, v_np)
    q_np, k_np, v_np = (x.float().cpu().numpy() for x in (q, k, v))
    wl = W.Workload("ragged", F, T, H, d, w, 3.0, 0, batch=B)
    plan = sfa.Plan(B, H, d, F, T, w, bound_limit=limit, bound_mode=1)
    out, ws = sfa.attention(plan, q, k, v)
    torch.cuda.synchronize()
    check_frame_stats(sfa, plan, ws, wl, q_np, k_np, 1, limit)
    ref = oracle.attention(q_np, k_np, v_np, F, T, w)
    assert_close(out.float().cpu().numpy(), ref, "frame bound ragged")


def _random_geoms(n=12, seed=777):
    g = np.random.default_rng(seed)
    return [(int(g.integers(0, 19)), 16 * int(g.integers(1, 11)), int(g.integers(0, 6)),
             int(g.integers(1, 4)), int(g.choice([64, 128])), int(g.integers(1, 3)),
             float(g.choice([40.0, 12.0, -1.0])), float(g.choice([1.0, 6.0])))
            for _ in range(n)]


@pytest.mark.parametrize("F,T,w,H,d,B,limit,boost", _random_geoms())
def test_frame_bound_random_geometries(sfa, F, T, w, H, d, B, limit, boost):
    """Seeded random geometries with the per-visible-frame bound; the last frame's keys
    optionally scaled up (outliers), limits that put some, all or no query frames online."""
    say(f"[frame_bound_random] F={F} T={T} w={w} H={H} d={d} B={B} limit={limit} "
        f"boost={boost}")
    S = (F + 1) * T
    g = np.random.default_rng(F * 313 + T * 7 + w + H + d + B)
    q_np = g.standard_normal((B, S, H, d)).astype(np.float32)
    k_np = (g.standard_normal((B, S, H, d)) + 3 * g.standard_normal((B, 1, H, d))).astype(
        np.float32)
    k_np[:, F * T:] *= boost
    v_np = g.standard_normal((B, S, H, d)).astype(np.float32)
    q, k, v = to_dev(q_np, k_np, v_np)
    q_np, k_np, v_np = (x.float().cpu().numpy() for x in (q, k, v))
    wl = W.Workload("random", F, T, H, d, w, 3.0, 0, batch=B)
    plan = sfa.Plan(B, H, d, F, T, w, bound_limit=limit, bound_mode=1)
    out, ws = sfa.attention(plan, q, k, v)
    torch.cuda.synchronize()
    check_frame_stats(sfa, plan, ws, wl, q_np, k_np, 1, limit)
    ref = oracle.attention(q_np, k_np, v_np, F, T, w)
    assert_close(out.float().cpu().numpy(), ref, "frame bound random")
