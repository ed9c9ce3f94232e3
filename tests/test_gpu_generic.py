"""GPU parity of the generic block-sparse ablation (sfa_generic_attention).

The ablation computes the same attention as the product path (section "Deleting
the mask" of "HeyGen x Google Cloud: Bringing Avatar IV to TPUs" describes it as
the starting point: generic tiles, element masks on partial blocks, the
reference frame as a second pass merged afterwards), so it must meet the same
tolerance against the oracle.
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


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_generic_full_parity(sfa, name):
    wl = W.ALL[name]
    say(f"[generic_full] {name}")
    q_np, k_np, v_np = W.make_inputs_np(wl)
    q, k, v = to_dev(q_np, k_np, v_np)
    plan = sfa.GenericPlan.for_workload(wl)
    out, _ = sfa.generic_attention(plan, q, k, v)
    torch.cuda.synchronize()
    ref = oracle.attention(q_np, k_np, v_np, wl.frames, wl.tokens_per_frame, wl.window)
    assert_close(out.float().cpu().numpy(), ref, f"generic {name}")


@pytest.mark.parametrize("F,T,w,H,d,B", [(0, 16, 0, 1, 64, 1), (3, 80, 5, 3, 128, 1),
                                         (6, 16, 1, 2, 64, 1), (2, 400, 1, 2, 128, 2),
                                         (13, 32, 2, 2, 128, 1)])
def test_generic_ragged(sfa, F, T, w, H, d, B):
    say(f"[generic_ragged] F={F} T={T} w={w} H={H} d={d} B={B}")
    S = (F + 1) * T
    g = np.random.default_rng(F * 100 + T + w)
    q_np = g.standard_normal((B, S, H, d)).astype(np.float32)
    k_np = (g.standard_normal((B, S, H, d)) + 3 * g.standard_normal((B, 1, H, d))).astype(
        np.float32)
    v_np = g.standard_normal((B, S, H, d)).astype(np.float32)
    q, k, v = to_dev(q_np, k_np, v_np)
    q_np, k_np, v_np = (x.float().cpu().numpy() for x in (q, k, v))
    plan = sfa.GenericPlan(B, H, d, F, T, w)
    out, _ = sfa.generic_attention(plan, q, k, v)
    torch.cuda.synchronize()
    ref = oracle.attention(q_np, k_np, v_np, F, T, w)
    assert_close(out.float().cpu().numpy(), ref, "generic ragged")


@pytest.mark.parametrize("name", ["720p", "stress"])
def test_generic_sampled_full_size(sfa, name):
    wl = W.ALL[name]
    say(f"[generic_sampled] {name}")
    q_np, k_np, v_np = W.make_inputs_np(wl)
    q, k, v = to_dev(q_np, k_np, v_np)
    plan = sfa.GenericPlan.for_workload(wl)
    out, _ = sfa.generic_attention(plan, q, k, v)
    torch.cuda.synchronize()
    T = wl.tokens_per_frame
    rows = set()
    for f in range(wl.frames + 1):
        rows.update({f * T, f * T + 100, (f + 1) * T - 1})
    rows.update({255, 256, 3583, 3584, wl.seq - 1})        # generic block edges
    rows = np.array(sorted(rows))
    got = out[0, torch.from_numpy(rows).cuda()].float().cpu().numpy()
    for h in (0, 3, wl.heads - 1):
        ref = oracle.attention_rows(q_np, k_np, v_np, wl.frames, T, wl.window, 0, h, rows)
        assert_close(got[:, h], ref, f"generic {name} head {h}")
    assert torch.isfinite(out.float()).all()


def _random_geoms(n=12, seed=4242):
    g = np.random.default_rng(seed)
    return [(int(g.integers(0, 19)), 16 * int(g.integers(1, 21)), int(g.integers(0, 6)),
             int(g.integers(1, 4)), int(g.choice([64, 128])), int(g.integers(1, 3)))
            for _ in range(n)]


@pytest.mark.parametrize("F,T,w,H,d,B", _random_geoms())
def test_generic_random_geometries(sfa, F, T, w, H, d, B):
    """Seeded random geometries: frame spans of 1-20 granules (rarely a multiple of the
    256 x 128 tiles, so most blocks near frame edges are partial), windows 0-5."""
    say(f"[generic_random] F={F} T={T} w={w} H={H} d={d} B={B}")
    S = (F + 1) * T
    g = np.random.default_rng(F * 131 + T * 17 + w + H + d + B)
    q_np = g.standard_normal((B, S, H, d)).astype(np.float32)
    k_np = (g.standard_normal((B, S, H, d)) + 3 * g.standard_normal((B, 1, H, d))).astype(
        np.float32)
    v_np = g.standard_normal((B, S, H, d)).astype(np.float32)
    q, k, v = to_dev(q_np, k_np, v_np)
    q_np, k_np, v_np = (x.float().cpu().numpy() for x in (q, k, v))
    plan = sfa.GenericPlan(B, H, d, F, T, w)
    out, _ = sfa.generic_attention(plan, q, k, v)
    torch.cuda.synchronize()
    ref = oracle.attention(q_np, k_np, v_np, F, T, w)
    assert_close(out.float().cpu().numpy(), ref, "generic random")
