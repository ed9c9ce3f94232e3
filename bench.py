"""Benchmark: one step = the whole hot path (prologue + attention kernel) over the
720p-shaped layer (reference frame + 13 frames x 3600 tokens, 12 heads, d = 128,
window +-2, batch 1) on one MI355X. Prints one JSON line.

value  = active-block TFLOP/s of the step: 4*d flops per visible (query, key)
         pair, divided by the wall time per step (sfa_norms + sfa_fwd).
roofline = the attention kernel alone (sfa_fwd is exactly one launch), timed
         with HIP events on its stream, against the bf16 dense MFMA peak;
         traffic = its HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE
         (profiles/), null if the kernel source changed since.
         measured_peak / pct_of_measured_peak = the same rate against chains of
         v_mfma_f32_32x32x16_bf16 with no memory traffic, timed live (libsfa_probe.so);
         loop_ceiling = the attention tile loop with its operands already in LDS (no
         HBM, no barriers), timed live: what this loop design can reach on the chip;
         sustained_clock_ghz = GRBM_GUI_ACTIVE cycles per XCD / kernel time from the
         committed rocprofv3 counters (profiles/), null if the kernel changed since.
cpu_baseline = the fp64 CPU oracle on a bounded sample of the same layer, blocks of up to
         1024 query rows of one (batch, head) per task over a pool of host threads.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "active-block attention TFLOP/s on 1 MI355X; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (no sparsity)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_kernel_720p_traffic.json")
KERNEL_SOURCES = ("sparse_attention_frame_amd/csrc/sfa_attn.h",
                  "sparse_attention_frame_amd/csrc/sfa_fwd.hip",
                  "sparse_attention_frame_amd/csrc/sfa_gfx950.h",
                  "sparse_attention_frame_amd/csrc/sfa_internal.h")
CLOCK_FILE = os.path.join(ROOT, "profiles", "fwd_kernel_720p_clock.json")
PRO_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prologue_kernel_720p_traffic.json")
PRO_SOURCES = ("sparse_attention_frame_amd/csrc/sfa_gfx950.h",
               "sparse_attention_frame_amd/csrc/sfa_prologue.hip",
               "sparse_attention_frame_amd/csrc/sfa_internal.h")


def kernel_source_hash(sources=KERNEL_SOURCES):
    """sha256 of the kernel sources' code: comments and blank space are dropped first, so
    a change to the comments alone leaves the profile records valid."""
    import hashlib
    import re

    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(path=TRAFFIC_FILE, sources=KERNEL_SOURCES, key="bytes_per_launch"):
    """A figure of the committed rocprofv3 counters (HBM bytes per kernel launch by
    default), or None when the kernel source changed since they were taken."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_hash(sources):
        return None
    return t.get(key)


def probe_ceilings():
    """Live matrix-core microbenchmarks (libsfa_probe.so), 8 waves per CU as the attention
    kernel runs: the MFMA-chain peak and the tile-loop ceilings, each the best of three
    launches. clock_ghz is the probe's own shader clock (s_memtime over s_memrealtime)."""
    from sparse_attention_frame_amd import probe

    out = {}
    for name, kind, iters in (("mfma_chain", probe.MFMA_CHAIN, 80000),
                              ("tile_loop_32rows", probe.TILE_LOOP, 40000),
                              ("tile_loop_64rows", probe.TILE_LOOP64, 20000),
                              ("tile_loop_32rows_no_softmax", probe.TILE_NOEXP, 40000)):
        r = max((probe.run(kind, waves=8, iters=iters) for _ in range(3)),
                key=lambda x: x["tflops"])   # best of three launches
        out[name] = {"tflops": round(r["tflops"], 1), "frac": round(r["tflops"] / PEAK_BF16_TFLOPS, 4),
                     "clock_ghz": round(r["clock_ghz"], 3), "mfma_busy": round(r["mfma_busy"], 3)}
    return out


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


def host_workers():
    """Threads for the CPU baseline: the cores this process may run on, capped by
    OMP_NUM_THREADS when set (a shared host grants one job a share of its cores)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_baseline(wl, q_np, k_np, v_np, out_gpu=None, gpu_stats=None, budget_s=12.0,
                 bound_limit=40.0, block=1024):
    """Time the oracle (as it stands) on blocks of up to `block` query rows inside one
    query frame (oracle.attention_block), one (batch, head, block) per task over a pool of
    host threads with one BLAS thread each, until about budget_s. With the GPU output
    ([B, S, H, d] float32) it also reports the parity of the rows done, and with the GPU's
    per-head statistics whether the eligibility flags match the oracle's."""
    import threading
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    T, F, d = wl.tokens_per_frame, wl.frames, wl.head_dim
    workers = host_workers()
    frames = [F // 2] + [f for f in range(F + 1) if f != F // 2]   # a full-window frame first
    tasks = [(b, h, r0, min(r0 + block, (f + 1) * T)) for b in range(wl.batch)
             for h in range(wl.heads) for f in frames for r0 in range(f * T, (f + 1) * T, block)]
    lock = threading.Lock()
    heads = {}
    done = []
    t0 = time.perf_counter()

    def one(task):
        if time.perf_counter() - t0 >= budget_s:
            return
        b, h, r0, r1 = task
        with lock:
            if (b, h) not in heads:
                heads[(b, h)] = tuple(np.ascontiguousarray(x[b, :, h, :], dtype=np.float64)
                                      for x in (q_np, k_np, v_np))
            qh, kh, vh = heads[(b, h)]
        ref = oracle.attention_block(qh, kh, vh, F, T, wl.window, r0, r1)
        with lock:
            done.append((task, ref, time.perf_counter()))

    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(workers) as ex:
        list(ex.map(one, tasks))
    if not done:
        return None
    dt = max(t for *_, t in done) - t0
    flops = sum(4.0 * d * (r1 - r0) * len(oracle.key_frames(r0 // T, F, wl.window)) * T
                for (_, _, r0, r1), *_ in done)
    rows = sum(r1 - r0 for (_, _, r0, r1), *_ in done)
    hs = sorted({(b, h) for (b, h, _, _), *_ in done})
    res = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": workers,
           "kind": "oracle", "cpu": cpu_model(),
           "sample": f"{len(done)} blocks of <= {block} query rows ({rows} rows) of (batch, head) "
                     f"{hs} of the {wl.name} layer, frame {F // 2} first, fp64 dense-masked "
                     f"numpy on {workers} threads, {dt:.1f} s"}
    if out_gpu is not None:
        # parity of the same rows in the same run (tolerance: max-abs 2e-2, rel-L2 5e-3)
        got = np.concatenate([out_gpu[b, r0:r1, h] for (b, h, r0, r1), _, _ in done])
        ref = np.concatenate([r for _, r, _ in done])
        diff = got.astype(np.float64) - ref
        res["parity"] = {"rows": int(len(ref)), "max_abs": float(np.abs(diff).max()),
                         "rel_l2": float(np.linalg.norm(diff) / np.linalg.norm(ref)),
                         "pass": bool(np.abs(diff).max() <= 2e-2
                                      and np.linalg.norm(diff) <= 5e-3 * np.linalg.norm(ref))}
    if gpu_stats is not None:
        # the eligibility flags must match bit for bit (untimed: after the sample)
        ref_st = oracle.head_stats(q_np, k_np, bound_limit=bound_limit)
        res["eligibility_match"] = bool(np.array_equal(np.asarray(gpu_stats["eligible"]),
                                                       ref_st["eligible"]))
    return res


def cpu_baseline_prologue(pw, x, gamma, w, cos, sin, outs=None, budget_s=12.0):
    """Time the oracle prologue on chunks of 512 tokens until ~budget_s; TFLOP/s. With the
    GPU's q, k, v it also reports the parity of the chunks done (tolerance of the tests:
    |got - ref| <= 1.2e-2 + 4e-3 |ref| element by element, rel-L2 <= 5e-3)."""
    import numpy as np

    import oracle

    flops_tok = 2.0 * pw.model_dim * 3 * pw.heads * pw.head_dim
    done, t0 = 0, time.perf_counter()
    worst, d2, r2 = -np.inf, 0.0, 0.0
    timed = 0.0
    while timed < budget_s and done < pw.seq:
        sl = slice(done, min(done + 512, pw.seq))
        t1 = time.perf_counter()
        refs = oracle.qkv_prologue(x[:, sl], gamma, w, cos[sl], sin[sl], pw.heads, pw.head_dim)
        timed += time.perf_counter() - t1
        if outs is not None:
            for got_t, ref in zip(outs, refs):
                got = got_t[:, sl].float().cpu().numpy().astype(np.float64)
                diff = np.abs(got - ref)
                worst = max(worst, float((diff - (1.2e-2 + 4e-3 * np.abs(ref))).max()))
                d2 += float((diff ** 2).sum())
                r2 += float((ref ** 2).sum())
        done = sl.stop
    res = {"value": round(done * pw.batch * flops_tok / timed / 1e12, 6), "unit": "TFLOP/s",
           "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)),
           "kind": "oracle", "cpu": cpu_model(),
           "sample": f"first {done} tokens of batch 0 in 512-token chunks, fp64, {timed:.1f} s"}
    if outs is not None:
        rl = (d2 / r2) ** 0.5
        res["parity"] = {"tokens": done, "rel_l2": rl, "pass": bool(worst <= 0 and rl <= 5e-3)}
    return res


def bench_prologue(args):
    """Fused prologue at the 720p layer's shape: x [1, 50400, 1536] bf16 -> q, k, v
    [1, 50400, 12, 128]. value = 2 * S * C * 3Hd flops / time of one sfa_qkv_prologue call
    (one kernel); the unfused PyTorch chain and torch's bare projection GEMM are timed
    beside."""
    import numpy as np
    import torch

    import sparse_attention_frame_amd as sfa
    from sparse_attention_frame_amd import workloads as W

    pw = W.PRO_720P
    log(f"bench: generating {pw.name} inputs")
    x_np, g_np, w_np, cos_np, sin_np = W.make_prologue_inputs_np(pw)
    dev = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
    x, gamma, w = bf(x_np), bf(g_np), bf(w_np)
    cos, sin = (torch.from_numpy(a).to(dev) for a in (cos_np, sin_np))
    stream = torch.cuda.current_stream()
    H, d, B, S, C = pw.heads, pw.head_dim, pw.batch, pw.seq, pw.model_dim
    wf = sfa.prologue_fold(w, gamma, stream=stream)
    q, k, v = sfa.qkv_prologue(x, wf, cos, sin, H, d, stream=stream)
    def step():
        sfa.qkv_prologue(x, wf, cos, sin, H, d, q=q, k=k, v=v, stream=stream)

    def unfused():
        xn = torch.nn.functional.rms_norm(x.float(), (C,), gamma.float(), 1e-6).to(torch.bfloat16)
        y = torch.nn.functional.linear(xn, w).view(B, S, 3, H, d)
        c, s_ = cos[None, :, None, :], sin[None, :, None, :]
        outs = []
        for i in range(3):
            u = y[:, :, i].float()
            if i < 2:
                a, b = u[..., :d // 2], u[..., d // 2:]
                u = torch.cat([a * c - b * s_, a * s_ + b * c], dim=-1)
            outs.append(u.to(torch.bfloat16).contiguous())
        return outs

    def timed(fn, n):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for e in ev:
            e[0].record(stream)
            fn()
            e[1].record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n, [a.elapsed_time(b) for a, b in ev]

    log("bench: warmup")
    for _ in range(args.warmup):
        step()
        unfused()
    log(f"bench: timing {args.steps} prologue calls")
    ms_step, ev_ms = timed(step, args.steps)
    un_ms, un_ev = timed(unfused, max(5, args.steps // 5))
    _, lin_ev = timed(lambda: torch.nn.functional.linear(x, w), max(5, args.steps // 5))
    ref = unfused()
    err = max(float((a.float() - b.float()).abs().max()) for a, b in zip((q, k, v), ref))
    flops = 2.0 * B * S * C * 3 * H * d
    kern_ms = float(np.mean(ev_ms))
    res = {
        "metric": "fused q/k/v prologue TFLOP/s on 1 MI355X; % of bf16 MFMA peak",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"720p-shaped layer prologue: x [{B}, {S}, {C}] -> q, k, v "
                               f"[{B}, {S}, {H}, {d}] (RMSNorm, projection, 3-axis rotary, "
                               "head packing)",
                   "gflop": round(flops / 1e9, 1)},
        "pct_of_peak": round(100.0 * flops / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "call_ms": round(kern_ms, 4), "call_min_ms": round(float(np.min(ev_ms)), 4),
        "unfused_torch_ms": round(float(np.mean(un_ev)), 4),
        "torch_linear_ms": round(float(np.mean(lin_ev)), 4),
        "max_abs_vs_unfused_torch": round(err, 5),
        "roofline": {"bound": "mfma", "kernel": "prologue_kernel (sfa_qkv_prologue is one "
                                                "launch)",
                     "achieved": round(flops / (kern_ms * 1e-3) / 1e12, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / (kern_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(PRO_TRAFFIC_FILE, PRO_SOURCES)},
    }
    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 2
        cx = torch.ones(n, dtype=torch.bfloat16, device=dev)
        cy = torch.empty_like(cx)
        torch.neg(cx, out=cy)        # reads and writes exactly copy_probe_mib MiB
        torch.cuda.synchronize()
        res["copy_probe_mib"] = args.copy_probe_mib
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline_prologue(pw, x_np, g_np, w_np, cos_np, sin_np,
                                                    outs=(q, k, v))
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="720p")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--waves", type=int, default=0, help="override waves per workgroup (4 or 8)")
    ap.add_argument("--block-q", type=int, default=0, help="override query rows per work item")
    ap.add_argument("--wave-rows", type=int, default=0,
                    help="override query rows per wave (32 or 64 with 8 waves)")
    ap.add_argument("--lds-stages", type=int, default=0, help="override K/V stages in flight")
    ap.add_argument("--key-split", type=int, default=0, choices=(0, -1),
                    help="0: the plan splits the tail items into two key halves; -1: never")
    ap.add_argument("--bound-mode", type=int, default=0,
                    help="0: per-head bound (default); 1: per-visible-frame bound")
    ap.add_argument("--bound-limit", type=float, default=40.0,
                    help="eligibility threshold of the fixed maximum (negative: every head online)")
    ap.add_argument("--head-groups", type=int, default=1,
                    help="split the heads into this many groups (sfa_attention_groups)")
    ap.add_argument("--group-streams", type=int, default=0,
                    help="streams the head groups are spread over (0: the current stream)")
    ap.add_argument("--ablation", choices=["none", "generic"], default="none",
                    help="generic: time the generic block-sparse two-pass ablation instead")
    ap.add_argument("--prologue", action="store_true",
                    help="time the fused q/k/v prologue (RMSNorm, projection, rotary, packing) "
                         "at the 720p layer's shape instead of the attention")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the live matrix-core microbenchmarks (measured peak, loop ceiling)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one elementwise copy of this size (calibrates HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.prologue:
        bench_prologue(args)
        return

    import numpy as np
    import torch

    import sparse_attention_frame_amd as sfa
    from sparse_attention_frame_amd import workloads as W

    wl = {**W.ALL, W.OUTLIER.name: W.OUTLIER}[args.workload]
    log(f"bench: generating {wl.name} inputs")
    q_np, k_np, v_np = W.make_inputs_np(wl)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (q_np, k_np, v_np))
    plan = sfa.Plan.for_workload(wl, waves=args.waves, block_q=args.block_q,
                                 lds_stages=args.lds_stages, bound_mode=args.bound_mode,
                                 bound_limit=args.bound_limit, key_split=args.key_split,
                                 wave_rows=args.wave_rows)
    ws = plan.workspace(dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    G = args.head_groups
    if G < 1 or wl.heads % G:
        print(f"--head-groups must divide the {wl.heads} heads", file=sys.stderr)
        sys.exit(2)
    if G > 1:
        gplan = sfa.Plan(wl.batch, wl.heads // G, wl.head_dim, wl.frames, wl.tokens_per_frame,
                         wl.window, waves=args.waves, block_q=args.block_q,
                         lds_stages=args.lds_stages, bound_mode=args.bound_mode,
                         bound_limit=args.bound_limit, key_split=args.key_split,
                         wave_rows=args.wave_rows)
        gws = torch.empty(G * gplan.info["workspace_bytes"], dtype=torch.uint8, device=dev)
        gstreams = [torch.cuda.Stream() for _ in range(args.group_streams)]

    if args.ablation == "generic":
        gen = sfa.GenericPlan.for_workload(wl)
        gen_ws = gen.workspace(dev)

    def step():
        if args.ablation == "generic":
            sfa.generic_attention(gen, q, k, v, out=out, workspace=gen_ws, stream=stream)
            return
        if G > 1:
            sfa.attention_groups(gplan, G, q, k, v, out=out, workspace=gws, streams=gstreams,
                                 stream=stream)
            return
        sfa.norms(plan, q, k, v, workspace=ws, stream=stream)
        sfa.fwd(plan, q, k, v, out=out, workspace=ws, stream=stream)

    log("bench: warmup")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        e[0].record(stream)
        if G > 1 or args.ablation != "none":   # one call: no prologue/kernel split
            e[1].record(stream)
            step()
        else:
            sfa.norms(plan, q, k, v, workspace=ws, stream=stream)
            e[1].record(stream)
            sfa.fwd(plan, q, k, v, out=out, workspace=ws, stream=stream)
        e[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    norms_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    fwd_all = [e[1].elapsed_time(e[2]) for e in ev]
    step_all = [e[0].elapsed_time(e[2]) for e in ev]
    fwd_ms = float(np.mean(fwd_all))
    fwd_min = float(np.min(fwd_all))

    info = plan.info
    flops = info["active_flops"]
    value = flops / (ms_step * 1e-3) / 1e12
    fwd_tf = flops / (fwd_ms * 1e-3) / 1e12   # with head groups: the whole grouped call
    if G > 1 or args.ablation != "none":
        sfa.norms(plan, q, k, v, workspace=ws, stream=stream)   # for the flag count below
    st = sfa.head_stats(plan, ws)
    fst = sfa.frame_stats(plan, ws)
    assert torch.isfinite(out.float()).all(), "non-finite output"

    traffic = measured_traffic()
    default_launch = (G == 1 and args.bound_mode == 0 and wl.name == "720p"
                      and args.bound_limit == 40.0 and args.ablation == "none"
                      and not (args.waves or args.block_q or args.lds_stages or args.key_split
                               or args.wave_rows))

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}-shaped layer: reference frame + F={wl.frames} frames x "
                               f"T={wl.tokens_per_frame} tokens (S={wl.seq}), H={wl.heads}, "
                               f"d={wl.head_dim}, window +-{wl.window}, batch {wl.batch}",
                   "block_q": info["block_q"], "waves": info["waves_per_item"],
                   "wave_rows": info["wave_rows"],
                   "items": info["items"], "split_frames": info["split_frames"],
                   "active_gflop": round(flops / 1e9, 1),
                   "eligible_heads": int(st["eligible"].sum()), "heads": wl.heads,
                   "bound_mode": args.bound_mode, "bound_limit": args.bound_limit,
                   "eligible_query_frames": int(fst["eligible"].sum()),
                   "query_frames": int(fst["eligible"].size),
                   "head_groups": G, "group_streams": args.group_streams,
                   "ablation": args.ablation},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_ms": round(fwd_ms, 4),
        "fwd_min_ms": round(fwd_min, 4),
        "fwd_median_ms": round(float(np.median(fwd_all)), 4),
        "step_event_median_ms": round(float(np.median(step_all)), 4),
        "step_event_min_ms": round(float(np.min(step_all)), 4),
        "norms_ms": round(norms_ms, 4),
        "roofline": {"bound": "mfma",
                     "kernel": ("whole step (generic two-pass ablation)" if args.ablation != "none"
                                else "fwd_kernel" if G == 1 else f"whole step ({G} head groups)"),
                     "achieved": round(fwd_tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic if default_launch else None,
                     "traffic_gbps": (round(traffic / (fwd_ms * 1e-3) / 1e9, 1)
                                      if default_launch and traffic else None),
                     "sustained_clock_ghz": (measured_traffic(CLOCK_FILE, key="clock_ghz")
                                             if default_launch else None)},
    }
    if wl.window >= wl.frames:
        # every video frame sees every frame: compare with dense attention over all S keys
        dense = 4.0 * wl.head_dim * float(wl.seq) ** 2 * wl.heads * wl.batch
        res["dense"] = {"gflop": round(dense / 1e9, 1),
                        "tflops_equiv": round(dense / (fwd_ms * 1e-3) / 1e12, 2),
                        "frac_of_peak": round(dense / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                        "note": "dense 4*d*S^2*H*B flops over the attention kernel's time"}
    if not args.no_probe:
        log("bench: matrix-core microbenchmarks")
        ceil = probe_ceilings()
        rf = res["roofline"]
        rf["measured_peak"] = {**ceil["mfma_chain"],
                               "probe": "independent v_mfma_f32_32x32x16_bf16 chains, 8 waves "
                                        "per CU, no memory (libsfa_probe.so)"}
        rf["pct_of_measured_peak"] = round(100.0 * fwd_tf / ceil["mfma_chain"]["tflops"], 2)
        rf["loop_ceiling"] = {k: v for k, v in ceil.items() if k != "mfma_chain"}
        rf["pct_of_loop_ceiling"] = round(100.0 * fwd_tf / ceil["tile_loop_32rows"]["tflops"], 2)
    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 2
        x = torch.ones(n, dtype=torch.bfloat16, device=dev)
        y = torch.empty_like(x)
        torch.neg(x, out=y)          # reads and writes exactly copy_probe_mib MiB
        torch.cuda.synchronize()
        res["copy_probe_mib"] = args.copy_probe_mib
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(wl, q_np, k_np, v_np, out.float().cpu().numpy(), st,
                                           bound_limit=args.bound_limit)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
