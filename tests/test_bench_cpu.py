"""bench.py pieces that need no GPU: the one-GPU guard, the traffic records' format, and the
cpu_baseline leg's parity and eligibility checks (fed the oracle's own output, and a corrupted
copy of it, so a broken comparison shows)."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import oracle  # noqa: E402
from sparse_attention_frame_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("path,sources", [(bench.TRAFFIC_FILE, bench.KERNEL_SOURCES),
                                          (bench.PRO_TRAFFIC_FILE, bench.PRO_SOURCES)])
def test_traffic_records_are_well_formed(path, sources):
    with open(path) as f:
        t = json.load(f)
    assert t["bytes_per_launch"] >= t["algorithmic_min_bytes"] > 0
    assert len(t["kernel_source_sha256"]) == 64
    assert all("rocprofv3 --pmc " in c and "bench.py" in c for c in t["commands"])
    # the FETCH_SIZE / WRITE_SIZE scales come from the copy probe of 1024 MiB (4 decimals)
    assert abs(t["fetch_scale"] * t["copy_fetch_kib"] / 1048576 - 1) < 1e-3
    assert abs(t["write_scale"] * t["copy_write_kib"] / 1048576 - 1) < 1e-3
    # bench reports the record only while the sources are the ones it was taken on
    current = bench.measured_traffic(path, sources)
    assert current in (None, t["bytes_per_launch"])


def test_clock_record_is_well_formed():
    with open(bench.CLOCK_FILE) as f:
        c = json.load(f)
    assert "GRBM_GUI_ACTIVE" in c["command"] and "rocprofv3 --pmc" in c["command"]
    assert abs(c["gui_cycles_per_xcd"] * c["xcds"] - c["grbm_gui_active_total"]) < 1.0
    # the clock is the cycles per XCD over the plain run's kernel time, below the 2.4 GHz peak
    assert abs(c["clock_ghz"] - c["gui_cycles_per_xcd"] / c["trace_average_ns"]) < 1e-3
    assert 0.5 < c["clock_ghz"] <= 2.4
    assert bench.measured_traffic(bench.CLOCK_FILE, key="clock_ghz") in (None, c["clock_ghz"])


def test_cpu_baseline_parity_and_eligibility_checks():
    wl = W.TINY
    q, k, v = W.make_inputs_np(wl)
    ref = oracle.attention(q, k, v, wl.frames, wl.tokens_per_frame, wl.window)
    flags = oracle.head_stats(q, k)["eligible"]
    good = bench.cpu_baseline(wl, q, k, v, ref.astype(np.float32), {"eligible": flags},
                              budget_s=5.0)
    assert good["kind"] == "oracle" and good["value"] > 0
    assert good["cores"] == bench.host_workers() >= 1
    # every (batch, head, frame) of the tiny layer fits the budget
    assert good["parity"]["rows"] == wl.batch * wl.heads * wl.seq
    assert good["parity"]["pass"] and good["eligibility_match"]
    bad_out = ref.astype(np.float32).copy()
    bad_out[0, (wl.frames // 2) * wl.tokens_per_frame + 5, 1, 3] += 0.1   # first frame timed
    bad = bench.cpu_baseline(wl, q, k, v, bad_out, {"eligible": ~flags}, budget_s=5.0)
    assert not bad["parity"]["pass"] and not bad["eligibility_match"]


def test_host_workers_honours_the_thread_cap(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    assert bench.host_workers() == min(3, len(os.sched_getaffinity(0)))
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.host_workers() == len(os.sched_getaffinity(0))


def test_cpu_baseline_prologue_parity_check():
    torch = pytest.importorskip("torch")
    pw = W.PRO_TINY
    x, g, w, c, s = W.make_prologue_inputs_np(pw)
    outs = [torch.from_numpy(t).to(torch.bfloat16)
            for t in oracle.qkv_prologue(x, g, w, c, s, pw.heads, pw.head_dim)]
    good = bench.cpu_baseline_prologue(pw, x, g, w, c, s, outs=outs, budget_s=0.2)
    assert good["parity"]["pass"]
    outs[1][0, 7, 2, 5] += 1.0
    bad = bench.cpu_baseline_prologue(pw, x, g, w, c, s, outs=outs, budget_s=0.2)
    assert not bad["parity"]["pass"]
