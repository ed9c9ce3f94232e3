"""GPU parity of the fused attention prologue (sfa_prologue_fold + sfa_qkv_prologue).

"HeyGen x Google Cloud: Bringing Avatar IV to TPUs", section "Layout as ABI"
(Fig. 5): normalisation, rotary embedding, projection and head packing run as
one kernel that writes the attention's input layout. The float64 oracle
(oracle.prologue) takes the same bf16 inputs.

Tolerance, derived from the arithmetic. The library folds gamma into the
weights in bf16 (relative rounding <= 2^-9 per weight, uniform, so the
projection picks up a random error of std ~ 2^-9 / sqrt(3) * |y|_rms ~ 1.1e-3 for
outputs of unit scale) and stores q, k, v in bf16 (<= 2^-9 |y|); fp32
accumulation and the fp32 rotation add ~1e-6. Hence, element by element,
|got - ref| <= 1.2e-2 + 4e-3 |ref| (the absolute term is ~10 standard
deviations of the fold error, the relative term twice the store rounding), and
over a tensor rel-L2 <= 5e-3 (expected ~1.6e-3). A wrong pairing, sign, head
or token moves entries by O(1).
"""
import sys
from dataclasses import replace

import numpy as np
import pytest

import oracle
from sparse_attention_frame_amd import workloads as W

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

ABS = 1.2e-2
REL = 4e-3
REL_L2 = 5e-3
ATT_MAX_ABS = 2e-2
ATT_REL_L2 = 5e-3


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def sfa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import sparse_attention_frame_amd as m

    m.lib()
    return m


def bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()


def f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def assert_close(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    worst = float((d - (ABS + REL * np.abs(ref))).max())
    rl = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    say(f"  {what}: max_abs={float(d.max()):.3e} rel_l2={rl:.3e}")
    assert worst <= 0 and rl <= REL_L2, (what, float(d.max()), rl)


def run(sfa, pw, x_np, gamma_np, w_np, cos, sin, x_pad=0, fused=False, eps=1e-6):
    """Device run; x_pad adds NaN columns after each row of x, fused writes q, k, v as views
    of one [B, S, 3, H, d] buffer."""
    B, S, C = x_np.shape
    H, d = pw.heads, pw.head_dim
    if x_pad:
        buf = np.full((B, S, C + x_pad), np.nan, np.float32)
        buf[:, :, :C] = x_np
        x = bf16_dev(buf)[:, :, :C]
    else:
        x = bf16_dev(x_np)
    wf = sfa.prologue_fold(bf16_dev(w_np), bf16_dev(gamma_np))
    outs = {}
    if fused:
        qkv = torch.full((B, S, 3, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        outs = dict(q=qkv[:, :, 0], k=qkv[:, :, 1], v=qkv[:, :, 2])
    q, k, v = sfa.qkv_prologue(x, wf, f32_dev(cos), f32_dev(sin), H, d, eps, **outs)
    torch.cuda.synchronize()
    return q, k, v


def check_against_oracle(q, k, v, pw, x_np, gamma_np, w_np, cos, sin, tokens=None, eps=1e-6):
    if tokens is not None:
        idx = torch.from_numpy(np.asarray(tokens)).cuda()
        q, k, v = (t[:, idx] for t in (q, k, v))
        x_np, cos, sin = x_np[:, tokens], cos[tokens], sin[tokens]
    rq, rk, rv = oracle.qkv_prologue(x_np, gamma_np, w_np, cos, sin, pw.heads, pw.head_dim, eps)
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        assert_close(got.float().cpu().numpy(), ref, f"{pw.name} {name}")


def test_fold_is_the_bf16_rounded_product(sfa):
    """Product of two bf16 values is exact in fp32, so the fold is one bf16 rounding."""
    say("[prologue_fold]")
    g = np.random.default_rng(7)
    for rows, cols in [(3, 64), (768, 256), (4608, 1536), (1, 2)]:
        w = bf16_dev(g.standard_normal((rows, cols)) * 0.05)
        gamma = bf16_dev(1.0 + 0.3 * g.standard_normal(cols))
        got = sfa.prologue_fold(w, gamma)
        torch.cuda.synchronize()
        ref = (gamma.cpu().float()[None, :] * w.cpu().float()).to(torch.bfloat16)
        assert torch.equal(got.cpu().view(torch.int16), ref.view(torch.int16)), (rows, cols)


@pytest.mark.parametrize("name", ["pro_tiny", "pro_small"])
def test_prologue_matches_oracle(sfa, name):
    pw = W.PROLOGUE[name]
    say(f"[prologue_full] {name} S={pw.seq} C={pw.model_dim} H={pw.heads} d={pw.head_dim}")
    x, gamma, w, cos, sin = W.make_prologue_inputs_np(pw)
    q, k, v = run(sfa, pw, x, gamma, w, cos, sin)
    check_against_oracle(q, k, v, pw, x, gamma, w, cos, sin)


@pytest.mark.parametrize("case", [
    dict(name="pro_tiny", batch=2),                         # two sequences, S < one tile
    dict(name="pro_tiny", batch=1, frames=0),               # one frame: S = 48
    dict(name="pro_tiny", batch=3, grid_h=1, grid_w=1, frames=0),   # S = 1
    dict(name="pro_small", batch=2, frames=2),              # ragged: S = 624
    dict(name="pro_tiny", heads=2, head_dim=128, model_dim=64),     # one K stage
    dict(name="pro_tiny", heads=8, head_dim=64, model_dim=192, frames=10),
    # more tiles than workgroups (each workgroup runs two or three, the next one's first
    # K stage fetched during the last stage of the one before): odd stage count ...
    dict(name="pro_tiny", heads=8, head_dim=64, model_dim=192, frames=31, grid_h=16, grid_w=43),
    # ... one K stage (no overlap, stage buffers alternate between tiles) ...
    dict(name="pro_tiny", heads=2, head_dim=128, model_dim=64, frames=31, grid_h=16, grid_w=43),
    # ... and d = 128 with five stages, 258 tiles (two workgroups take a second one)
    dict(name="pro_tiny", heads=4, head_dim=128, model_dim=320, frames=15, grid_h=16, grid_w=43),
])
def test_prologue_shapes(sfa, case):
    case = dict(case)
    pw = replace(W.PROLOGUE[case.pop("name")], **case)
    say(f"[prologue_shapes] {pw}")
    x, gamma, w, cos, sin = W.make_prologue_inputs_np(pw)
    q, k, v = run(sfa, pw, x, gamma, w, cos, sin)
    check_against_oracle(q, k, v, pw, x, gamma, w, cos, sin)


def test_prologue_strided_input_and_fused_output(sfa):
    """x rows padded with NaN columns, q/k/v written as views of one [B, S, 3, H, d] buffer:
    the padding is never read and every output element is written."""
    pw = replace(W.PRO_SMALL, batch=2, frames=3)
    say(f"[prologue_strided] {pw}")
    x, gamma, w, cos, sin = W.make_prologue_inputs_np(pw)
    q, k, v = run(sfa, pw, x, gamma, w, cos, sin, x_pad=64, fused=True)
    for t in (q, k, v):
        assert torch.isfinite(t.float()).all()
    check_against_oracle(q, k, v, pw, x, gamma, w, cos, sin)


def test_prologue_zero_rows_and_eps(sfa):
    """A token whose hidden state is zero projects to exactly zero; eps enters the RMS."""
    pw = W.PRO_TINY
    say("[prologue_zero_rows]")
    x, gamma, w, cos, sin = W.make_prologue_inputs_np(pw)
    x[0, [0, 17, pw.seq - 1]] = 0.0
    x[0, 5] *= 1e-3                      # eps is comparable to mean(x^2) here
    eps = 1e-5
    q, k, v = run(sfa, pw, x, gamma, w, cos, sin, eps=eps)
    for t in (q, k, v):
        assert (t[0, [0, 17, pw.seq - 1]].float() == 0).all()
    check_against_oracle(q, k, v, pw, x, gamma, w, cos, sin, eps=eps)


def test_prologue_720p_sampled(sfa):
    """Full 720p hidden states (50400 x 1536 -> 12 heads x 128), tokens sampled at tile,
    frame and sequence edges."""
    pw = W.PRO_720P
    say(f"[prologue_720p] S={pw.seq}")
    x, gamma, w, cos, sin = W.make_prologue_inputs_np(pw)
    q, k, v = run(sfa, pw, x, gamma, w, cos, sin)
    for t in (q, k, v):
        assert torch.isfinite(t.float()).all()
    T = pw.tokens_per_frame
    toks = {0, 1, 255, 256, 257, 511, 512, pw.seq - 256, pw.seq - 1, pw.seq - 2}
    for f in range(pw.frames + 1):
        toks.update({f * T, f * T + 81, (f + 1) * T - 1})
    g = np.random.default_rng(3)
    toks.update(g.integers(0, pw.seq, 256).tolist())
    check_against_oracle(q, k, v, pw, x, gamma, w, cos, sin, tokens=np.array(sorted(toks)))


def test_prologue_feeds_attention(sfa):
    """The prologue's outputs are the attention's inputs as they stand: the chain
    prologue -> sfa_attention matches the oracle's attention of those bf16 tensors, and the
    float64 chain of the two oracles within the attention tolerance."""
    pw = replace(W.PRO_SMALL, frames=6)
    window = 2
    say(f"[prologue_chain] {pw} w={window}")
    x, gamma, w, cos, sin = W.make_prologue_inputs_np(pw)
    q, k, v = run(sfa, pw, x, gamma, w, cos, sin)
    plan = sfa.Plan(pw.batch, pw.heads, pw.head_dim, pw.frames, pw.tokens_per_frame, window)
    out, _ = sfa.attention(plan, q, k, v)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    qn, kn, vn = (t.float().cpu().numpy() for t in (q, k, v))
    ref = oracle.attention(qn, kn, vn, pw.frames, pw.tokens_per_frame, window)
    rq, rk, rv = oracle.qkv_prologue(x, gamma, w, cos, sin, pw.heads, pw.head_dim)
    ref64 = oracle.attention(rq, rk, rv, pw.frames, pw.tokens_per_frame, window)
    for what, r in (("attention of prologue outputs", ref), ("float64 chain", ref64)):
        dd = got - r
        mx = float(np.abs(dd).max())
        rl = float(np.linalg.norm(dd) / np.linalg.norm(r))
        say(f"  {what}: max_abs={mx:.3e} rel_l2={rl:.3e}")
        assert mx <= ATT_MAX_ABS and rl <= ATT_REL_L2, (what, mx, rl)


def test_layer_step_graph_replays_match_eager(sfa):
    """Fused prologue, then norm pass and attention, captured once into a HIP graph and
    replayed three times with eager work and a synchronisation between the replays: every
    replay reproduces the eager q, k, v and output bit for bit."""
    pw = replace(W.PRO_SMALL, frames=6)
    window = 2
    say(f"[layer_graph] {pw} w={window}")
    x, gamma, w, cos, sin = W.make_prologue_inputs_np(pw)
    H, d = pw.heads, pw.head_dim
    xd, cd, sd = bf16_dev(x), f32_dev(cos), f32_dev(sin)
    wf = sfa.prologue_fold(bf16_dev(w), bf16_dev(gamma))
    q, k, v = sfa.qkv_prologue(xd, wf, cd, sd, H, d)
    plan = sfa.Plan(pw.batch, H, d, pw.frames, pw.tokens_per_frame, window)
    ws = plan.workspace()
    out = torch.empty_like(q)

    def step():
        sfa.qkv_prologue(xd, wf, cd, sd, H, d, q=q, k=k, v=v)
        sfa.attention(plan, q, k, v, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (q, k, v, out)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (q, k, v, out):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, r in zip((q, k, v, out), ref):
            assert torch.equal(got, r), rep


def _random_shapes(n=10, seed=99):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(g.choice([64, 128]))
        heads = int(g.choice([4, 8, 12])) if d == 64 else int(g.choice([2, 4, 6]))
        out.append(dict(name="pro_tiny", batch=int(g.integers(1, 3)), frames=int(g.integers(0, 12)),
                        grid_h=int(g.integers(1, 20)), grid_w=int(g.integers(1, 30)),
                        heads=heads, head_dim=d, model_dim=64 * int(g.integers(1, 9))))
    return out


@pytest.mark.parametrize("case", _random_shapes())
def test_prologue_random_shapes(sfa, case):
    """Seeded random shapes: any sequence length (ragged last token tile), 1-8 K stages,
    d 64 / 128, one or two sequences."""
    case = dict(case)
    pw = replace(W.PROLOGUE[case.pop("name")], **case)
    say(f"[prologue_random] {pw}")
    x, gamma, w, cos, sin = W.make_prologue_inputs_np(pw)
    q, k, v = run(sfa, pw, x, gamma, w, cos, sin)
    check_against_oracle(q, k, v, pw, x, gamma, w, cos, sin)
