"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Tolerance for bf16 inputs with fp32 accumulation: max |O_gpu - O_oracle| <= 2e-2
and ||O_gpu - O_oracle||_2 / ||O_oracle||_2 <= 5e-3; the per-head eligibility
flag of the fixed-maximum path must match the oracle exactly.
"""
import os
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

    m.lib()  # raises if libsfa.so is missing: no fallback path exists
    return m


def to_dev(*xs):
    return [torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda() for x in xs]


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    return float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(ref))


def assert_close(got, ref, what):
    mx, rl = errors(got, ref)
    say(f"  {what}: max_abs={mx:.3e} rel_l2={rl:.3e}")
    assert mx <= MAX_ABS and rl <= REL_L2, (what, mx, rl)


def run(sfa, wl_like, q, k, v, **plan_kw):
    plan = sfa.Plan(*wl_like, **plan_kw)
    out, ws = sfa.attention(plan, q, k, v)
    torch.cuda.synchronize()
    return plan, out, ws


def geom(wl):
    return (wl.batch, wl.heads, wl.head_dim, wl.frames, wl.tokens_per_frame, wl.window)


def check_stats(sfa, plan, ws, q_np, k_np, bound_limit=40.0):
    st = sfa.head_stats(plan, ws)
    ref = oracle.head_stats(q_np, k_np, bound_limit=bound_limit)
    np.testing.assert_array_equal(st["eligible"], ref["eligible"])
    np.testing.assert_allclose(st["kmax"], ref["kmax"], rtol=1e-4)
    np.testing.assert_allclose(st["qmax"], ref["qmax"], rtol=1e-5)
    np.testing.assert_allclose(st["bound"], ref["bound"], rtol=1e-4)
    np.testing.assert_allclose(st["mu"], ref["mu"], rtol=0, atol=1e-4 * (1 + np.abs(ref["mu"]).max()))
    return st, ref


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_parity_full(sfa, name):
    wl = W.ALL[name]
    say(f"[parity_full] {name}")
    q_np, k_np, v_np = W.make_inputs_np(wl)
    q, k, v = to_dev(q_np, k_np, v_np)
    plan, out, ws = run(sfa, geom(wl), q, k, v)
    ref = oracle.attention(q_np, k_np, v_np, wl.frames, wl.tokens_per_frame, wl.window)
    assert_close(out.float().cpu().numpy(), ref, name)
    st, ref_st = check_stats(sfa, plan, ws, q_np, k_np)
    assert st["eligible"].all()
    # per-row half of the norm array
    qn, qmu = sfa.row_norms(plan, ws)
    qd = q_np.astype(np.float64)
    np.testing.assert_allclose(qn, np.sqrt((qd ** 2).sum(-1)).transpose(0, 2, 1), rtol=1e-5)
    np.testing.assert_allclose(qmu, np.einsum("bshd,bhd->bhs", qd, ref_st["mu"]), rtol=0,
                               atol=1e-3)


def sample_rows(wl, block_q=512, n_random=24, seed=0):
    T, S = wl.tokens_per_frame, wl.seq
    rows = set()
    last = (T - 1) // block_q * block_q    # first row of the frame's last (ragged) block
    for f in range(wl.frames + 1):
        # frame edges, granule, wave-tile and block edges, the ragged last block of the frame
        rows.update({f * T, f * T + 15, f * T + 16, f * T + 31, f * T + 32, f * T + 63,
                     f * T + 64, f * T + 255, f * T + 256, f * T + T // 2,
                     f * T + block_q - 1, f * T + block_q, f * T + last - 1, f * T + last,
                     (f + 1) * T - 17, (f + 1) * T - 16, (f + 1) * T - 1})
    rows = {r for r in rows if 0 <= r < S}
    g = np.random.default_rng(seed)
    rows.update(int(x) for x in g.integers(0, S, n_random))
    return np.array(sorted(rows))


def oracle_heads(q_np, k_np, v_np, wl, heads, block=1024, workers=None):
    """Every row of the chosen heads of batch 0 from the oracle, computed as blocks of at
    most `block` rows inside one query frame (oracle.attention_block) on a thread pool
    with one BLAS thread per worker. Returns {head: float64 [S, d]}."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    T = wl.tokens_per_frame
    per_head = {h: tuple(np.ascontiguousarray(x[0, :, h, :], dtype=np.float64)
                         for x in (q_np, k_np, v_np)) for h in heads}
    out = {h: np.empty((wl.seq, wl.head_dim)) for h in heads}
    jobs = [(h, r0, min(r0 + block, (f + 1) * T)) for h in heads
            for f in range(wl.frames + 1) for r0 in range(f * T, (f + 1) * T, block)]

    def work(job):
        h, r0, r1 = job
        qh, kh, vh = per_head[h]
        out[h][r0:r1] = oracle.attention_block(qh, kh, vh, wl.frames, T, wl.window, r0, r1)

    workers = workers or max(1, min(16, os.cpu_count() or 1))
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(workers) as ex:
        list(ex.map(work, jobs))
    return out


# whole heads compared at full size: one fixed-maximum head, and on the stress layers one
# head of the online path too
FULL_HEADS = {"720p": (0,), "1080p": (0,), "stress": (0, 3), "stress_w13": (0, 3)}


@pytest.mark.parametrize("name", ["720p", "1080p", "stress", "stress_w13"])
def test_parity_sampled_full_size(sfa, name):
    """Full-size inputs in the benchmark's launch configuration: every row of whole heads
    (FULL_HEADS) and sampled rows of every other head."""
    wl = W.ALL[name]
    say(f"[parity_sampled] {name} generating inputs")
    q_np, k_np, v_np = W.make_inputs_np(wl)
    q, k, v = to_dev(q_np, k_np, v_np)
    say(f"[parity_sampled] {name} launching")
    plan, out, ws = run(sfa, geom(wl), q, k, v)
    st, _ = check_stats(sfa, plan, ws, q_np, k_np)
    expect_bad = set(wl.boost_heads)
    assert {h for h in range(wl.heads) if not st["eligible"][0, h]} == expect_bad
    rows = sample_rows(wl, plan.info["block_q"])
    got_all = out[0, torch.from_numpy(rows).cuda()].float().cpu().numpy()   # [R, H, d]
    for h in range(wl.heads):
        if h in FULL_HEADS[name]:
            continue
        ref = oracle.attention_rows(q_np, k_np, v_np, wl.frames, wl.tokens_per_frame, wl.window,
                                    0, h, rows)
        assert_close(got_all[:, h], ref, f"{name} head {h} ({len(rows)} rows)")
    assert torch.isfinite(out.float()).all()
    say(f"[parity_sampled] {name} oracle on whole heads {FULL_HEADS[name]}")
    full = oracle_heads(q_np, k_np, v_np, wl, FULL_HEADS[name])
    got = out[0].float().cpu().numpy()
    for h, ref in full.items():
        assert_close(got[:, h], ref, f"{name} head {h} (all {wl.seq} rows)")
        # and frame by frame, so no frame hides behind the others
        T = wl.tokens_per_frame
        for f in range(wl.frames + 1):
            assert_close(got[f * T:(f + 1) * T, h], ref[f * T:(f + 1) * T],
                         f"{name} head {h} frame {f}")


@pytest.mark.parametrize("limit", [40.0, -1.0])
def test_parity_sampled_d64_batch2_many_items(sfa, limit):
    """d = 64, two sequences, 576 work items (more than one per workgroup, so the
    persistent workgroups' queues, stealing and counter reset run for this head size too),
    both softmax paths; sampled rows of every (batch, head)."""
    F, T, w, H, d, B = 13, 720, 2, 6, 64, 2
    say(f"[d64_batch2] limit={limit}")
    S = (F + 1) * T
    g = np.random.default_rng(64)
    q_np = g.standard_normal((B, S, H, d)).astype(np.float32)
    k_np = (g.standard_normal((B, S, H, d)) + 3 * g.standard_normal((B, 1, H, d))).astype(
        np.float32)
    v_np = g.standard_normal((B, S, H, d)).astype(np.float32)
    q, k, v = to_dev(q_np, k_np, v_np)
    q_np, k_np, v_np = (x.float().cpu().numpy() for x in (q, k, v))
    plan, out, ws = run(sfa, (B, H, d, F, T, w), q, k, v, bound_limit=limit)
    # 256-row query blocks: 256, 256 and a ragged 208 per frame
    assert plan.info["block_q"] == 256
    assert plan.info["items"] == B * H * (F + 1 + plan.info["split_frames"]) * 3
    st, _ = check_stats(sfa, plan, ws, q_np, k_np, bound_limit=limit)
    assert st["eligible"].all() == (limit > 0)
    rows = np.array(sorted({f * T + r for f in range(F + 1)
                            for r in (0, 31, 32, 255, 256, 511, 512, 687, 688, 703, 704,
                                      T - 1)}
                           | set(g.integers(0, S, 16).tolist())))
    got_all = out[:, torch.from_numpy(rows).cuda()].float().cpu().numpy()   # [B, R, H, d]
    for b in range(B):
        for h in range(H):
            ref = oracle.attention_rows(q_np, k_np, v_np, F, T, w, b, h, rows)
            assert_close(got_all[b, :, h], ref, f"b {b} head {h} ({len(rows)} rows)")
    assert torch.isfinite(out.float()).all()


def test_full_size_frame_indicator_has_no_mass_outside_window(sfa):
    """720p shape, every row: with v_j = one-hot(frame(j)) the output is exactly zero on
    frames outside the row's window and sums to ~1 (any size, no oracle needed)."""
    wl = W.P720
    say("[frame_indicator] 720p")
    q_np, k_np, _ = W.make_inputs_np(wl)
    q, k = to_dev(q_np, k_np)
    T, F = wl.tokens_per_frame, wl.frames
    v = torch.zeros_like(q)
    frame = torch.arange(wl.seq, device="cuda") // T
    v[0, torch.arange(wl.seq, device="cuda"), :, frame] = 1.0
    plan, out, _ = run(sfa, geom(wl), q, k, v)
    o = out[0, :, :, :F + 1].float()                               # [S, H, F+1]
    allowed = torch.from_numpy(oracle.mask_matrix(F, 1, wl.window)).cuda()  # frame level
    outside = ~allowed[frame]                                      # [S, F+1]
    assert (o[outside.unsqueeze(1).expand_as(o)] == 0).all()
    assert (o[(~outside).unsqueeze(1).expand_as(o)] > 0).all()
    assert torch.allclose(o.sum(-1), torch.ones_like(o[..., 0]), atol=1e-2)
    assert (out[0, :, :, F + 1:] == 0).all()


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_forced_online_path(sfa, name):
    wl = W.ALL[name]
    say(f"[forced_online] {name}")
    q_np, k_np, v_np = W.make_inputs_np(wl)
    q, k, v = to_dev(q_np, k_np, v_np)
    plan, out, ws = run(sfa, geom(wl), q, k, v, bound_limit=-1.0)
    st = sfa.head_stats(plan, ws)
    assert not st["eligible"].any()
    ref = oracle.attention(q_np, k_np, v_np, wl.frames, wl.tokens_per_frame, wl.window)
    assert_close(out.float().cpu().numpy(), ref, f"{name} online")


# (F, T, w, H, d, B): tails of 1, 2 and 3 granules, a lone granule, reference frame only,
# window 0, window past both ends, batch 2, d = 64 and 128, 5-granule query blocks
RAGGED = [(0, 16, 0, 1, 64, 1), (1, 16, 0, 2, 128, 1), (2, 48, 1, 2, 64, 2), (3, 80, 5, 3, 128, 1),
          (6, 48, 1, 2, 128, 1), (5, 32, 2, 1, 64, 1), (4, 112, 1, 2, 128, 2), (9, 16, 3, 4, 128, 1)]


@pytest.mark.parametrize("F,T,w,H,d,B", RAGGED)
@pytest.mark.parametrize("limit", [40.0, -1.0])
def test_ragged_geometries(sfa, F, T, w, H, d, B, limit):
    say(f"[ragged] F={F} T={T} w={w} H={H} d={d} B={B} limit={limit}")
    S = (F + 1) * T
    g = np.random.default_rng(F * 1000 + T + w)
    q_np = g.standard_normal((B, S, H, d)).astype(np.float32)
    k_np = (g.standard_normal((B, S, H, d)) + 3 * g.standard_normal((B, 1, H, d))).astype(
        np.float32)
    v_np = g.standard_normal((B, S, H, d)).astype(np.float32)
    q, k, v = to_dev(q_np, k_np, v_np)
    q_np, k_np, v_np = (x.float().cpu().numpy() for x in (q, k, v))
    plan, out, ws = run(sfa, (B, H, d, F, T, w), q, k, v, bound_limit=limit)
    ref = oracle.attention(q_np, k_np, v_np, F, T, w)
    assert_close(out.float().cpu().numpy(), ref, "ragged")
    check_stats(sfa, plan, ws, q_np, k_np, bound_limit=limit)


@pytest.mark.parametrize("limit", [40.0, -1.0])
def test_largest_frame_count(sfa, limit):
    """1024 frame slots (reference + 1023 frames), the most a plan takes: the per-frame
    tables at full size, on the fixed-maximum path and forced online. Sampled rows of the
    first, last and some random frames against the oracle."""
    F, T, w, H, d = 1023, 16, 2, 2, 64
    say(f"[largest_frame_count] F={F} limit={limit}")
    S = (F + 1) * T
    g = np.random.default_rng(1023)
    q_np = g.standard_normal((1, S, H, d)).astype(np.float32)
    k_np = (g.standard_normal((1, S, H, d)) + 3 * g.standard_normal((1, 1, H, d))).astype(
        np.float32)
    v_np = g.standard_normal((1, S, H, d)).astype(np.float32)
    q, k, v = to_dev(q_np, k_np, v_np)
    q_np, k_np, v_np = (x.float().cpu().numpy() for x in (q, k, v))
    plan, out, ws = run(sfa, (1, H, d, F, T, w), q, k, v, bound_limit=limit)
    st, _ = check_stats(sfa, plan, ws, q_np, k_np, bound_limit=limit)
    assert st["eligible"].all() == (limit > 0)
    frames = sorted({*range(4), *range(F - 3, F + 1), *g.integers(4, F - 3, 24).tolist()})
    rows = np.array([f * T + r for f in frames for r in (0, 7, T - 1)])
    got = out[0, torch.from_numpy(rows).cuda()].float().cpu().numpy()
    for h in range(H):
        ref = oracle.attention_rows(q_np, k_np, v_np, F, T, w, 0, h, rows)
        assert_close(got[:, h], ref, f"head {h} ({len(rows)} rows)")
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("limit", [40.0, -1.0])
def test_long_frames(sfa, limit):
    """Frames of 65536 tokens (4096 granules each; an item of a middle frame streams 12288
    key granules through its LDS stages, 768 stages of 64 keys), window +-1, a ragged last
    block in no frame but key halves on the end frames: sampled rows of every frame against
    the oracle, on the fixed-maximum path and forced online."""
    F, T, w, H, d = 7, 65536, 1, 1, 128
    say(f"[long_frames] T={T} limit={limit}")
    S = (F + 1) * T
    g = np.random.default_rng(65536)
    q_np = g.standard_normal((1, S, H, d)).astype(np.float32)
    k_np = (g.standard_normal((1, S, H, d)) + 3 * g.standard_normal((1, 1, H, d))).astype(
        np.float32)
    v_np = g.standard_normal((1, S, H, d)).astype(np.float32)
    q, k, v = to_dev(q_np, k_np, v_np)
    q_np, k_np, v_np = (x.float().cpu().numpy() for x in (q, k, v))
    plan, out, ws = run(sfa, (1, H, d, F, T, w), q, k, v, bound_limit=limit)
    st, _ = check_stats(sfa, plan, ws, q_np, k_np, bound_limit=limit)
    assert st["eligible"].all() == (limit > 0)
    bq = plan.info["block_q"]
    rows = np.array(sorted({f * T + r for f in range(F + 1)
                            for r in (0, 31, 32, bq - 1, bq, T // 2 + 5, T - bq, T - 1)}))
    got = out[0, torch.from_numpy(rows).cuda()].float().cpu().numpy()
    ref = oracle.attention_rows(q_np, k_np, v_np, F, T, w, 0, 0, rows)
    assert_close(got[:, 0], ref, f"{len(rows)} rows")
    assert torch.isfinite(out.float()).all()


def test_zero_query_gives_window_mean(sfa):
    F, T, w, H, d = 6, 48, 1, 2, 128
    say("[zero_query]")
    S = (F + 1) * T
    g = np.random.default_rng(3)
    v_np = g.standard_normal((1, S, H, d)).astype(np.float32)
    k_np = g.standard_normal((1, S, H, d)).astype(np.float32)
    q, k, v = to_dev(np.zeros_like(v_np), k_np, v_np)
    plan, out, _ = run(sfa, (1, H, d, F, T, w), q, k, v)
    vv = v.float().cpu().numpy().astype(np.float64)
    got = out.float().cpu().numpy()
    for f in range(F + 1):
        frames = [0] if f == 0 else [0] + [x for x in range(f - w, f + w + 1) if 1 <= x <= F]
        mean = np.mean(np.concatenate([vv[0, x * T:(x + 1) * T] for x in frames]), axis=0)
        assert_close(got[0, f * T:(f + 1) * T], np.broadcast_to(mean, (T, H, d)), f"frame {f}")


def staged_reference(x, d):
    """The staged layouts of sfa_norms restated on the host from a [B, S, H, d] array
    (uint16 bf16 bit patterns): K as [granule][8-element chunk][16 keys][8] and V as
    [granule][d][16 keys] with the 8-key halves of row e swapped when (e / 8) is odd."""
    B, S, H, _ = x.shape
    G = S // 16
    xt = x.transpose(0, 2, 1, 3).reshape(B, H, G, 16, d)          # [b, h, g, key, e]
    k = xt.reshape(B, H, G, 16, d // 8, 8).transpose(0, 1, 2, 4, 3, 5)
    v = xt.transpose(0, 1, 2, 4, 3).reshape(B, H, G, d, 2, 8)     # [b, h, g, e, half, 8]
    swap = ((np.arange(d) >> 3) & 1).astype(bool)
    v = v.copy()
    v[:, :, :, swap] = v[:, :, :, swap][:, :, :, :, ::-1]
    return k.reshape(B, H, S * d), v.reshape(B, H, S * d)


def test_double_run_is_bitwise_identical(sfa):
    """Two runs of one build must agree bit for bit before differences are trusted: the
    output and every array the prologue writes for the kernel (head and per-frame stats,
    row norms, staged K and V), read through the ABI; the staged copies are exactly the
    inputs in the documented layouts."""
    wl = W.SMALL
    say("[determinism] small")
    q, k, v = to_dev(*W.make_inputs_np(wl))
    _, a, wa = run(sfa, geom(wl), q, k, v)
    _, b, wb = run(sfa, geom(wl), q, k, v)
    assert torch.equal(a, b)
    # the defined parts of the workspace (sections are padded to 256 bytes)
    pa = sfa.Plan(*geom(wl))
    sa, sb = sfa.head_stats(pa, wa), sfa.head_stats(pa, wb)
    for key in sa:
        np.testing.assert_array_equal(sa[key], sb[key])
    fa, fb = sfa.frame_stats(pa, wa), sfa.frame_stats(pa, wb)
    for key in fa:
        np.testing.assert_array_equal(fa[key], fb[key])
    for x, y in zip(sfa.row_norms(pa, wa), sfa.row_norms(pa, wb)):
        np.testing.assert_array_equal(x, y)
    ka, va = sfa.staged(pa, wa)
    kb, vb = sfa.staged(pa, wb)
    np.testing.assert_array_equal(ka, kb)
    np.testing.assert_array_equal(va, vb)
    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    kr, _ = staged_reference(bits(k), wl.head_dim)
    _, vr = staged_reference(bits(v), wl.head_dim)
    np.testing.assert_array_equal(ka, kr)
    np.testing.assert_array_equal(va, vr)


@pytest.mark.parametrize("name", ["small", "720p"])
def test_work_queue_covers_every_item_on_repeated_launches(sfa, name):
    """The attention kernel runs persistent workgroups that take items from per-XCD
    counters in the workspace (zeroed by sfa_norms, reset by the last workgroup of each
    launch). A workspace full of garbage, then three launches after one sfa_norms, each
    into an output full of NaN: every element is written, identically each time."""
    wl = W.ALL[name]
    say(f"[work queue] {name}")
    q, k, v = to_dev(*W.make_inputs_np(wl))
    plan = sfa.Plan(*geom(wl))
    ws = plan.workspace()
    ws.fill_(0xFF)
    sfa.norms(plan, q, k, v, workspace=ws)
    first = None
    for _ in range(3):
        out = torch.full_like(q, float("nan"))
        sfa.fwd(plan, q, k, v, out=out, workspace=ws)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
        if first is None:
            first = out
        else:
            assert torch.equal(out, first)


def test_head_subset_and_layouts_are_bitwise_equal(sfa):
    """Head groups see exactly the same mask; strided layouts change nothing."""
    wl = W.SMALL
    say("[layouts] small")
    q, k, v = to_dev(*W.make_inputs_np(wl))
    _, full, _ = run(sfa, geom(wl), q, k, v)
    # a group of heads as strided views of the full tensors
    sub = (wl.batch, 3, wl.head_dim, wl.frames, wl.tokens_per_frame, wl.window)
    _, part, _ = run(sfa, sub, q[:, :, 2:5], k[:, :, 2:5], v[:, :, 2:5])
    assert torch.equal(part, full[:, :, 2:5])
    # BHSD storage viewed as [B, S, H, d]
    qh, kh, vh = (x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for x in (q, k, v))
    assert qh.stride(2) == wl.seq * wl.head_dim
    plan = sfa.Plan(*geom(wl))
    ws = plan.workspace()
    outh = torch.empty_like(qh)
    sfa.attention(plan, qh, kh, vh, out=outh, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(outh, full)


def test_error_paths_on_device(sfa):
    wl = W.TINY
    q, k, v = to_dev(*W.make_inputs_np(wl))
    plan = sfa.Plan(*geom(wl))
    bad = torch.empty(q.numel() + 8, dtype=torch.bfloat16, device="cuda")[4:4 + q.numel()]
    bad = bad.view(q.shape)
    with pytest.raises(sfa.SfaError) as e:
        sfa.attention(plan, bad, k, v)
    assert e.value.status == -2
    small_ws = torch.empty(plan.info["workspace_bytes"] - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(sfa.SfaError) as e:
        sfa.attention(plan, q, k, v, workspace=small_ws)
    assert e.value.status == -1
    with pytest.raises(ValueError):
        sfa.attention(plan, q[:, :-16], k, v)


@pytest.mark.parametrize("name,groups,nstreams", [("small", 1, 0), ("small", 2, 2),
                                                  ("small", 4, 3), ("small", 8, 4),
                                                  ("720p", 3, 3)])
def test_head_groups_are_bitwise_equal(sfa, name, groups, nstreams):
    """Head groups on their own streams (section "Hiding collectives": heads are
    independent) match the oracle (every element on the small layer, sampled rows of every
    head, hence of every group, at 720p) and give exactly the single-launch result."""
    wl = W.ALL[name]
    say(f"[head_groups] {name} groups={groups} streams={nstreams}")
    q_np, k_np, v_np = W.make_inputs_np(wl)
    q, k, v = to_dev(q_np, k_np, v_np)
    _, full, _ = run(sfa, geom(wl), q, k, v)
    gp = sfa.Plan(wl.batch, wl.heads // groups, wl.head_dim, wl.frames, wl.tokens_per_frame,
                  wl.window)
    streams = [torch.cuda.Stream() for _ in range(nstreams)]
    for rep in range(2):
        out, _ = sfa.attention_groups(gp, groups, q, k, v, streams=streams)
        torch.cuda.synchronize()
        assert torch.equal(out, full), rep
    if name == "small":
        ref = oracle.attention(q_np, k_np, v_np, wl.frames, wl.tokens_per_frame, wl.window)
        assert_close(out.float().cpu().numpy(), ref, f"groups={groups}")
    else:
        rows = sample_rows(wl, gp.info["block_q"])
        got = out[0, torch.from_numpy(rows).cuda()].float().cpu().numpy()
        for h in range(wl.heads):
            ref = oracle.attention_rows(q_np, k_np, v_np, wl.frames, wl.tokens_per_frame,
                                        wl.window, 0, h, rows)
            assert_close(got[:, h], ref, f"groups={groups} group {h // gp.geometry.heads} "
                                         f"head {h}")


@pytest.mark.parametrize("name", ["small", "720p"])
def test_graph_replays_match_eager(sfa, name):
    """One step (sfa_norms + sfa_fwd) captured into a HIP graph and replayed three times,
    with eager work and a synchronisation between the replays: every replay writes the
    eager result bit for bit (the work-queue counters are cleared by a kernel inside the
    step, not by a memset)."""
    wl = W.ALL[name]
    say(f"[graph] {name}")
    q, k, v = to_dev(*W.make_inputs_np(wl))
    plan = sfa.Plan(*geom(wl))
    ws = plan.workspace()
    out = torch.empty_like(q)
    sfa.attention(plan, q, k, v, out=out, workspace=ws)  # eager, outside the capture
    torch.cuda.synchronize()
    ref = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sfa.attention(plan, q, k, v, out=out, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        ws[: ws.numel() // 2].fill_(0xA5)  # eager work on the workspace between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep


# (B, H, d, F, T, w): the small workload, and d = 64 with two sequences and 5-granule frames
OPTION_GEOMS = [(1, 8, 128, 8, 208, 2), (2, 2, 64, 6, 80, 1)]


@pytest.mark.parametrize("geom_", OPTION_GEOMS)
@pytest.mark.parametrize("opts", [dict(waves=8, lds_stages=2), dict(waves=8, lds_stages=4),
                                  dict(waves=4, lds_stages=2), dict(waves=4, lds_stages=3),
                                  dict(waves=4, lds_stages=4), dict(block_q=16),
                                  dict(block_q=48), dict(block_q=48, waves=4),
                                  dict(block_q=112), dict(block_q=112, lds_stages=2),
                                  dict(block_q=48, lds_stages=4),
                                  dict(key_split=-1), dict(wave_rows=32),
                                  dict(wave_rows=32, lds_stages=4),
                                  dict(wave_rows=32, block_q=112), dict(block_q=176),
                                  dict(block_q=80, lds_stages=2), dict(wave_rows=64),
                                  dict(wave_rows=64, block_q=176),
                                  dict(wave_rows=64, lds_stages=2), dict(waves=12),
                                  dict(waves=12, lds_stages=2), dict(waves=12, block_q=112),
                                  dict(waves=12, block_q=80)])
@pytest.mark.parametrize("limit", [40.0, -1.0])
def test_plan_options_parity(sfa, geom_, opts, limit):
    """Every launch configuration sfa_plan_create_ex offers (8 waves of one or two query
    tiles, 4 waves of two, two to four LDS stages, one-granule query blocks, query blocks
    that do not divide the frame so that its last block is ragged and some waves hold no
    real row or only one real query tile, no key split), both softmax paths, against the
    oracle."""
    B, H, d, F, T, w = geom_
    say(f"[plan_options] {geom_} {opts} limit={limit}")
    S = (F + 1) * T
    g = np.random.default_rng(B * 100 + T)
    q_np = g.standard_normal((B, S, H, d)).astype(np.float32)
    k_np = (g.standard_normal((B, S, H, d)) + 3 * g.standard_normal((B, 1, H, d))).astype(
        np.float32)
    v_np = g.standard_normal((B, S, H, d)).astype(np.float32)
    q, k, v = to_dev(q_np, k_np, v_np)
    q_np, k_np, v_np = (x.float().cpu().numpy() for x in (q, k, v))
    plan, out, ws = run(sfa, geom_, q, k, v, bound_limit=limit, **opts)
    if "block_q" in opts:
        assert plan.info["block_q"] == min(opts["block_q"], T)
    if "waves" in opts:
        assert plan.info["waves_per_item"] == opts["waves"]
    if "wave_rows" in opts:
        assert plan.info["wave_rows"] == opts["wave_rows"]
    ref = oracle.attention(q_np, k_np, v_np, F, T, w)
    assert_close(out.float().cpu().numpy(), ref, "options")
    check_stats(sfa, plan, ws, q_np, k_np, bound_limit=limit)


def _random_cases(n=24, seed=2024):
    """Seeded geometries and plan options: frames 0-18, 1-10 granules per frame, windows 0-5
    (also past both ends), 1-3 heads, d 64 / 128, one or two sequences, any launch option."""
    g = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        F = int(g.integers(0, 19))
        T = 16 * int(g.integers(1, 11))
        w = int(g.integers(0, 6))
        H = int(g.integers(1, 4))
        d = int(g.choice([64, 128]))
        B = int(g.integers(1, 3))
        waves = int(g.choice([0, 4, 8, 12]))
        stages = int(g.choice([0, 2, 3, 4]))
        limit = float(g.choice([40.0, -1.0, 40.0]))
        rows = 0 if waves == 4 else int(g.choice([0, 32, 64]))
        if waves == 12:                      # 96-key stages: 32 rows per wave, <= 3 stages
            rows, stages = 32, min(stages, 3)
        cases.append((F, T, w, H, d, B, waves, stages, limit, rows))
    return cases


@pytest.mark.parametrize("F,T,w,H,d,B,waves,stages,limit,rows", _random_cases())
def test_random_geometries_and_options(sfa, F, T, w, H, d, B, waves, stages, limit, rows):
    say(f"[random] F={F} T={T} w={w} H={H} d={d} B={B} waves={waves} stages={stages} "
        f"limit={limit} wave_rows={rows}")
    S = (F + 1) * T
    g = np.random.default_rng(F * 7919 + T * 31 + w * 7 + H + d + B)
    q_np = g.standard_normal((B, S, H, d)).astype(np.float32)
    k_np = (g.standard_normal((B, S, H, d)) + 3 * g.standard_normal((B, 1, H, d))).astype(
        np.float32)
    v_np = g.standard_normal((B, S, H, d)).astype(np.float32)
    q, k, v = to_dev(q_np, k_np, v_np)
    q_np, k_np, v_np = (x.float().cpu().numpy() for x in (q, k, v))
    plan, out, ws = run(sfa, (B, H, d, F, T, w), q, k, v, bound_limit=limit, waves=waves,
                        lds_stages=stages, wave_rows=rows)
    ref = oracle.attention(q_np, k_np, v_np, F, T, w)
    assert_close(out.float().cpu().numpy(), ref, "random")
    check_stats(sfa, plan, ws, q_np, k_np, bound_limit=limit)


@pytest.mark.parametrize("limit", [40.0, -1.0])
@pytest.mark.parametrize("rows,waves", [(0, 0), (64, 8), (32, 12)])
def test_key_split_halves_merge(sfa, limit, rows, waves):
    """The items of the cheapest multi-frame query frames run as two key halves merged by
    whichever finishes second: both paths match the oracle, the merged rows agree with the
    unsplit run to rounding, rows of the other frames are bitwise those of the unsplit run,
    and two runs are bitwise identical whatever the finishing order."""
    F, T, w, H, d, B = 9, 240, 2, 4, 128, 2
    say(f"[key_split] limit={limit} wave_rows={rows} waves={waves}")
    S = (F + 1) * T
    g = np.random.default_rng(91)
    q_np = g.standard_normal((B, S, H, d)).astype(np.float32)
    k_np = (g.standard_normal((B, S, H, d)) + 3 * g.standard_normal((B, 1, H, d))).astype(
        np.float32)
    v_np = g.standard_normal((B, S, H, d)).astype(np.float32)
    q, k, v = to_dev(q_np, k_np, v_np)
    q_np, k_np, v_np = (x.float().cpu().numpy() for x in (q, k, v))
    plan, a, _ = run(sfa, (B, H, d, F, T, w), q, k, v, bound_limit=limit, wave_rows=rows,
                     waves=waves)
    assert plan.info["split_frames"] == 2        # frames 1 and F see 4 frames, the fewest
    _, b, _ = run(sfa, (B, H, d, F, T, w), q, k, v, bound_limit=limit, wave_rows=rows,
                  waves=waves)
    assert torch.equal(a, b)
    _, whole, _ = run(sfa, (B, H, d, F, T, w), q, k, v, bound_limit=limit, key_split=-1,
                      wave_rows=rows, waves=waves)
    ref = oracle.attention(q_np, k_np, v_np, F, T, w)
    assert_close(a.float().cpu().numpy(), ref, "split")
    assert_close(whole.float().cpu().numpy(), ref, "whole")
    split_rows = torch.zeros(S, dtype=torch.bool)
    split_rows[T:2 * T] = True
    split_rows[F * T:] = True
    assert torch.equal(a[:, ~split_rows.cuda()], whole[:, ~split_rows.cuda()])
    diff = (a[:, split_rows.cuda()].float() - whole[:, split_rows.cuda()].float()).abs().max()
    assert float(diff) <= 2e-2
