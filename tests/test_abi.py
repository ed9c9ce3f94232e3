"""C-ABI checks that need no GPU: exports, planning, work order and argument errors.

Planning follows "HeyGen x Google Cloud: Bringing Avatar IV to TPUs", section
"Deleting the mask": query blocks lie inside one frame, key ranges are whole
frames (reference + window), so the plan's ranges expanded to tokens must
equal the oracle's mask exactly.
"""
import ctypes
import json
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from sparse_attention_frame_amd import _lib
from sparse_attention_frame_amd import workloads as W
from sparse_attention_frame_amd.api import Plan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sfa.h")


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sfa_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    declared = _declared_functions()
    assert declared, "no declarations parsed"
    assert sorted(_lib.EXPORTS) == declared
    for name in declared:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (sfa_[a-z_]+)\b", out))
    assert set(declared) <= exported


def test_probe_library_exports_its_header():
    """libsfa_probe.so (the microbenchmarks the benchmark reports against) exports what
    include/sfa_probe.h declares; the calls need a GPU and are not made here."""
    from sparse_attention_frame_amd import probe

    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "sfa_probe.h")).read(),
                  flags=re.S)
    declared = sorted(set(re.findall(r"\b(sfa_[a-z_]+)\s*\(", text)))
    assert declared == sorted(probe.EXPORTS)
    pl = probe.lib()
    assert pl.sfa_probe_scratch_bytes() >= 1024 * 512 * 4
    out = subprocess.run(["nm", "-D", "--defined-only", probe.PROBE_LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    assert set(declared) <= set(re.findall(r"\bT (sfa_[a-z_]+)\b", out))
    r = probe.Result()
    # argument checks come before any HIP call
    assert pl.sfa_probe_run(9, 8, 10, None, 0, None, r) == -1
    assert pl.sfa_probe_run(0, 6, 10, None, 0, None, r) == -1


def test_status_strings(L):
    for st in (0, -1, -2, -3, -4):
        assert L.sfa_status_str(st)
    assert b"unknown" in L.sfa_status_str(7)


def _auto_block(T, slots, wave_rows=64, waves=8, target=256):
    """The default block size, restated: one workgroup's rows (waves x wave_rows) or the
    whole frame when it is shorter; when that gives fewer than `target` work items (slots
    per block index x blocks per frame), the most blocks per frame that keep the items at
    `target` or fewer, of balanced size (ceil(T / n) rounded up to 16 rows), but at least
    one wave's rows."""
    top = min(T, waves * wave_rows)
    if top <= wave_rows:
        return top
    if slots * -(-T // top) >= target:
        return top
    n = target // slots
    bq = 16 * -(-(T // 16) // n)
    return min(max(bq, wave_rows), top)


@pytest.mark.parametrize("name,block_q", [("tiny", 32), ("small", 112), ("720p", 256),
                                          ("1080p", 256), ("stress", 256)])
def test_plan_query_blocks_cover_the_frame(L, name, block_q):
    wl = W.ALL[name]
    p = Plan.for_workload(wl)
    T = wl.tokens_per_frame
    slots = wl.batch * wl.heads * (wl.frames + 1 + p.info["split_frames"])
    assert block_q == _auto_block(T, slots, wave_rows=32)
    assert p.info["wave_rows"] == 32
    nqb = -(-T // block_q)
    assert p.info["block_q"] == block_q and block_q % 16 == 0
    # blocks of block_q rows, the last one ragged: a frame costs ceil(T / 32) wave tiles
    assert (nqb - 1) * block_q < T <= nqb * block_q
    assert p.info["granule"] == 16
    # the query frames seeing the fewest frames (more than one) run as two key halves
    vis = [len(oracle.key_frames(f, wl.frames, wl.window)) for f in range(1, wl.frames + 1)]
    vmin = min([v for v in vis if v >= 2], default=0)
    assert p.info["split_frames"] == sum(v == vmin for v in vis)
    assert p.info["items"] == wl.batch * wl.heads * (wl.frames + 1 + p.info["split_frames"]) * nqb
    off = Plan.for_workload(wl, key_split=-1)
    assert off.info["split_frames"] == 0
    off_slots = wl.batch * wl.heads * (wl.frames + 1)
    assert off.info["block_q"] == _auto_block(T, off_slots, wave_rows=32)
    assert off.info["items"] == off_slots * -(-T // off.info["block_q"])


def test_active_pairs_match_oracle_and_golden(L):
    with open(os.path.join(ROOT, "tests", "golden", "frame_pairs.json")) as f:
        gold = json.load(f)
    for name, wl in W.ALL.items():
        p = Plan.for_workload(wl)
        T = wl.tokens_per_frame
        assert p.info["active_pairs"] == gold[name]["pairs"] * T * T * wl.heads * wl.batch
        assert p.info["active_flops"] == 4.0 * wl.head_dim * p.info["active_pairs"]
    for wl in (W.TINY, W.SMALL):
        p = Plan.for_workload(wl)
        m = oracle.mask_matrix(wl.frames, wl.tokens_per_frame, wl.window)
        assert p.info["active_pairs"] == int(m.sum()) * wl.heads * wl.batch


@pytest.mark.parametrize("F,T,w", [(4, 48, 1), (8, 208, 2), (13, 32, 2), (13, 32, 13), (5, 16, 0),
                                   (0, 16, 3), (1, 16, 0), (6, 16, 1)])
def test_key_ranges_expand_to_the_oracle_mask(L, F, T, w):
    p = Plan(1, 1, 64, F, T, w)
    mask = oracle.mask_matrix(F, T, w)
    for f in range(F + 1):
        ranges = p.key_ranges(f)
        assert 1 <= len(ranges) <= 2
        row = np.zeros(mask.shape[1], dtype=bool)
        for a, b in ranges:
            assert a % T == 0 and b % T == 0 and a < b
            row[a:b] = True
        if len(ranges) == 2:
            assert ranges[0][1] < ranges[1][0]   # adjacent ranges are merged
        for i in range(f * T, (f + 1) * T):
            np.testing.assert_array_equal(mask[i], row)


@pytest.mark.parametrize("B,H,F,T,w,bq", [(1, 12, 13, 3600, 2, 0), (2, 3, 4, 48, 1, 16),
                                          (1, 5, 7, 64, 3, 32), (3, 2, 0, 32, 0, 0),
                                          (1, 16, 13, 3600, 13, 0), (2, 2, 5, 208, 1, 112),
                                          (1, 3, 3, 48, 2, 32)])
@pytest.mark.parametrize("key_split", [0, -1])
def test_work_items_cover_everything_once_largest_first(L, B, H, F, T, w, bq, key_split):
    """Every (batch, head, frame, query block) is covered exactly once: by one item that
    sees all of the frame's keys, or by two key halves whose ranges are disjoint and
    together give exactly those keys; items come largest first (cost = key frames)."""
    p = Plan(B, H, 128, F, T, w, block_q=bq, key_split=key_split)
    n = p.info["items"]
    nqb = -(-T // p.info["block_q"])
    nsplit = p.info["split_frames"]
    assert n == B * H * (F + 1 + nsplit) * nqb
    items = [p.item(i) for i in range(n)]
    keys = [p.item_keys(i) for i in range(n)]
    seen = {}
    for (b, h, f, qb), (half, ranges) in zip(items, keys):
        assert 0 <= b < B and 0 <= h < H and 0 <= f <= F and 0 <= qb < nqb
        seen.setdefault((b, h, f, qb), []).append((half, ranges))
    assert len(seen) == B * H * (F + 1) * nqb
    split_frames = set()
    for (b, h, f, qb), parts in seen.items():
        frames = np.zeros(F + 1, dtype=np.int32)   # key frames covered, with multiplicity
        for half, ranges in parts:
            for a, e in ranges:
                assert a % T == 0 and e % T == 0 and a < e
                frames[a // T:e // T] += 1
        assert sorted(hf for hf, _ in parts) in ([-1], [0, 1])
        if len(parts) == 2:
            split_frames.add(f)
        want = np.zeros(F + 1, dtype=np.int32)
        want[oracle.key_frames(f, F, w)] = 1
        np.testing.assert_array_equal(frames, want)
    assert len(split_frames) == nsplit
    cost = [sum(e - a for a, e in r) // T for (_, r) in keys]
    run = 8 * nqb
    full = n // run * run
    # whole runs of 8 groups: every run costs no more than the one before
    for r0 in range(0, full - run, run):
        assert min(cost[r0:r0 + run]) >= max(cost[r0 + run:r0 + 2 * run])
        # XCD x (blocks r0 + x, r0 + x + 8, ...) serves one (batch, head, frame) group
        for x in range(8):
            assert len({items[i][:3] for i in range(r0 + x, r0 + run, 8)}) == 1
    assert sorted(cost, reverse=True)[0] == cost[0]


def _geom(**kw):
    g = dict(batch=1, heads=2, head_dim=64, frames=4, tokens_per_frame=48, window=1,
             scale=0.0, bound_limit=40.0)
    g.update(kw)
    return _lib.Geometry(**g)


@pytest.mark.parametrize("kw,status", [
    (dict(tokens_per_frame=40), _lib.SFA_ERR_UNSUPPORTED),
    (dict(head_dim=96), _lib.SFA_ERR_UNSUPPORTED),
    (dict(window=-1), _lib.SFA_ERR_INVALID),
    (dict(frames=-1), _lib.SFA_ERR_INVALID),
    (dict(batch=0), _lib.SFA_ERR_INVALID),
    (dict(heads=0), _lib.SFA_ERR_INVALID),
    (dict(scale=-1.0), _lib.SFA_ERR_INVALID),
    (dict(scale=float("nan")), _lib.SFA_ERR_INVALID),
    (dict(frames=2000), _lib.SFA_ERR_UNSUPPORTED),
    (dict(frames=1024), _lib.SFA_ERR_UNSUPPORTED),
])
def test_invalid_geometry(L, kw, status):
    h = ctypes.c_void_p(123)
    assert L.sfa_plan_create(ctypes.byref(_geom(**kw)), ctypes.byref(h)) == status
    assert h.value is None


def test_largest_frame_count_is_accepted(L):
    # 1024 frame slots (reference + 1023 frames) is the largest per-frame table
    h = ctypes.c_void_p()
    assert L.sfa_plan_create(ctypes.byref(_geom(frames=1023, tokens_per_frame=16)),
                             ctypes.byref(h)) == _lib.SFA_OK
    assert h.value is not None
    L.sfa_plan_destroy(h)


def test_tile_override_errors(L):
    h = ctypes.c_void_p()
    g = _geom()
    for bq in (8, 24, 528, -16):     # not a multiple of 16, too large, negative
        opt = _lib.PlanOptions(bq, 0, 0)
        assert L.sfa_plan_create_ex(ctypes.byref(g), ctypes.byref(opt), ctypes.byref(h)) == \
            _lib.SFA_ERR_UNSUPPORTED, bq
    for bq, want in ((32, 32), (96, 48), (256, 48)):   # ragged last block; at most the frame
        opt = _lib.PlanOptions(bq, 0, 0)
        assert L.sfa_plan_create_ex(ctypes.byref(g), ctypes.byref(opt), ctypes.byref(h)) == 0
        info = _lib.PlanInfo()
        assert L.sfa_plan_get_info(h, ctypes.byref(info)) == 0
        assert info.block_q == want, bq
        L.sfa_plan_destroy(h)
    for waves in (1, 2, 6, 16, -4):
        opt = _lib.PlanOptions(0, waves, 0)
        assert L.sfa_plan_create_ex(ctypes.byref(g), ctypes.byref(opt), ctypes.byref(h)) == \
            _lib.SFA_ERR_UNSUPPORTED, waves
    for stages in (1, 5, -2):
        opt = _lib.PlanOptions(0, 0, stages)
        assert L.sfa_plan_create_ex(ctypes.byref(g), ctypes.byref(opt), ctypes.byref(h)) == \
            _lib.SFA_ERR_UNSUPPORTED, stages
    for mode in (2, -1, 7):
        opt = _lib.PlanOptions(0, 0, 0, mode)
        assert L.sfa_plan_create_ex(ctypes.byref(g), ctypes.byref(opt), ctypes.byref(h)) == \
            _lib.SFA_ERR_UNSUPPORTED, mode
    for mode in (0, 1):
        opt = _lib.PlanOptions(0, 0, 0, mode)
        assert L.sfa_plan_create_ex(ctypes.byref(g), ctypes.byref(opt), ctypes.byref(h)) == 0
        info = _lib.PlanInfo()
        assert L.sfa_plan_get_info(h, ctypes.byref(info)) == 0
        assert info.bound_mode == mode
        L.sfa_plan_destroy(h)
    # the default block of this 10-group geometry: the frame (48 rows) does not give 256
    # items, so one wave's rows (32; 64 with 4 waves, cut to the frame)
    for bq, waves, want in ((16, 0, 16), (48, 4, 48), (0, 8, 32), (0, 4, 48), (0, 12, 32)):
        opt = _lib.PlanOptions(bq, waves, 3)
        assert L.sfa_plan_create_ex(ctypes.byref(g), ctypes.byref(opt), ctypes.byref(h)) == 0
        info = _lib.PlanInfo()
        assert L.sfa_plan_get_info(h, ctypes.byref(info)) == 0
        assert info.block_q == want and info.waves_per_item == (waves or 8)
        assert info.wave_rows == (64 if waves == 4 else 32)
        L.sfa_plan_destroy(h)
    # rows per wave: 32 or 64 with 8 waves, only 64 with 4; the block is at most
    # waves x rows per wave
    for waves, rows, ok in ((8, 32, True), (8, 64, True), (0, 32, True), (4, 64, True),
                            (12, 32, True), (4, 32, False), (12, 64, False), (8, 16, False),
                            (8, 128, False), (0, -32, False)):
        opt = _lib.PlanOptions(0, waves, 0, 0, 0, rows)
        # 64 heads x 5 frames: the default block is the largest, one workgroup's rows
        st = L.sfa_plan_create_ex(ctypes.byref(_geom(heads=64, tokens_per_frame=1024)),
                                  ctypes.byref(opt), ctypes.byref(h))
        assert st == (0 if ok else _lib.SFA_ERR_UNSUPPORTED), (waves, rows)
        if ok:
            info = _lib.PlanInfo()
            assert L.sfa_plan_get_info(h, ctypes.byref(info)) == 0
            assert info.wave_rows == rows and info.block_q == (waves or 8) * rows
            L.sfa_plan_destroy(h)
    opt = _lib.PlanOptions(0, 12, 4)                # 96-key stages: at most three fit in LDS
    assert L.sfa_plan_create_ex(ctypes.byref(_geom()), ctypes.byref(opt), ctypes.byref(h)) == \
        _lib.SFA_ERR_UNSUPPORTED
    opt = _lib.PlanOptions(512, 8, 0, 0, 0, 32)     # more rows than 8 waves of 32 hold
    assert L.sfa_plan_create_ex(ctypes.byref(_geom(tokens_per_frame=1024)), ctypes.byref(opt),
                                ctypes.byref(h)) == _lib.SFA_ERR_UNSUPPORTED
    assert L.sfa_plan_create_ex(ctypes.byref(g), None, ctypes.byref(h)) == 0
    L.sfa_plan_destroy(h)
    assert L.sfa_plan_create(None, ctypes.byref(h)) == _lib.SFA_ERR_INVALID
    assert L.sfa_plan_create(ctypes.byref(g), None) == _lib.SFA_ERR_INVALID


def test_call_validation_happens_before_any_launch(L):
    """Argument errors are reported without touching the GPU (this runs on CPU)."""
    p = Plan(1, 2, 64, 4, 48, 1)
    S = p.seq
    good = _lib.Tensor(4096, S * 2 * 64, 2 * 64, 64)
    ws = ctypes.c_void_p(1 << 20)
    need = p.info["workspace_bytes"]
    assert L.sfa_norms(p.handle, good, good, good, None, need, None) == _lib.SFA_ERR_INVALID
    assert L.sfa_norms(p.handle, good, good, good, ws, need - 1, None) == _lib.SFA_ERR_INVALID
    assert L.sfa_norms(None, good, good, good, ws, need, None) == _lib.SFA_ERR_INVALID
    bad_ptr = _lib.Tensor(4096 + 8, S * 128, 128, 64)
    assert L.sfa_norms(p.handle, bad_ptr, good, good, ws, need, None) == _lib.SFA_ERR_UNSUPPORTED
    bad_stride = _lib.Tensor(4096, S * 128, 130, 64)
    assert L.sfa_norms(p.handle, good, bad_stride, good, ws, need, None) == \
        _lib.SFA_ERR_UNSUPPORTED
    assert L.sfa_norms(p.handle, good, good, bad_stride, ws, need, None) == \
        _lib.SFA_ERR_UNSUPPORTED
    huge_stride = _lib.Tensor(4096, S * (1 << 25), 1 << 25, 64)
    assert L.sfa_norms(p.handle, good, huge_stride, good, ws, need, None) == \
        _lib.SFA_ERR_UNSUPPORTED
    null_t = _lib.Tensor(None, S * 128, 128, 64)
    assert L.sfa_fwd(p.handle, good, good, good, null_t, ws, need, None) == _lib.SFA_ERR_INVALID
    # output aliasing an input is refused
    assert L.sfa_fwd(p.handle, good, good, good, good, ws, need, None) == _lib.SFA_ERR_INVALID
    mis_ws = ctypes.c_void_p((1 << 20) + 16)
    assert L.sfa_fwd(p.handle, good, good, good, _lib.Tensor(1 << 30, S * 128, 128, 64), mis_ws,
                     need, None) == _lib.SFA_ERR_UNSUPPORTED


def test_read_calls_check_the_workspace_size(L):
    """The sfa_read_* calls refuse a null or too-small workspace before copying anything
    (the copies would read past the allocation); this runs on CPU."""
    p = Plan(1, 2, 64, 4, 48, 1)
    need = p.info["workspace_bytes"]
    ws = ctypes.c_void_p(1 << 20)
    f = (ctypes.c_float * 4096)()
    u8 = (ctypes.c_uint8 * 64)()
    u16 = (ctypes.c_uint16 * 64)()
    for size, wsp in ((need - 1, ws), (0, ws), (need, None)):
        assert L.sfa_read_head_stats(p.handle, wsp, size, f, f, f, f, u8, None) == \
            _lib.SFA_ERR_INVALID
        assert L.sfa_read_row_norms(p.handle, wsp, size, f, f, None) == _lib.SFA_ERR_INVALID
        assert L.sfa_read_frame_stats(p.handle, wsp, size, f, f, u8, None) == \
            _lib.SFA_ERR_INVALID
        assert L.sfa_read_staged(p.handle, wsp, size, u16, u16, None) == _lib.SFA_ERR_INVALID
    assert L.sfa_read_staged(None, ws, need, u16, u16, None) == _lib.SFA_ERR_INVALID


def test_static_entry_refuses_before_any_launch(L):
    """sfa_attention_static checks the plan against its fixed 64 MiB workspace before it
    touches the GPU (this runs on CPU): the 720p-shaped layer needs more."""
    p = Plan.for_workload(W.ALL["720p"])
    assert p.info["workspace_bytes"] > 64 << 20
    t = _lib.Tensor(4096, 1 << 12, 128, 0)
    assert L.sfa_attention_static(p.handle, t, t, t, t, None) == _lib.SFA_ERR_TOO_LARGE
    assert L.sfa_attention_static(None, t, t, t, t, None) == _lib.SFA_ERR_INVALID
    assert b"64 MiB" in L.sfa_status_str(_lib.SFA_ERR_TOO_LARGE)


def test_bound_limit_cap(L):
    """bound_limit above 126 / (2 log2 e) would let the largest weight of a row underflow
    on the fixed-maximum path; the plan refuses it (negative limits force the online
    path and stay valid)."""
    cap = 126.0 / (2.0 * np.log2(np.e))
    h = ctypes.c_void_p()
    for lim, want in ((40.0, 0), (43.66, 0), (-1.0, 0), (-1e30, 0), (43.68, -2), (100.0, -2),
                      (float("inf"), -2), (float("nan"), -1)):
        st = L.sfa_plan_create(ctypes.byref(_geom(bound_limit=lim)), ctypes.byref(h))
        assert st == want, (lim, st)
        if st == 0:
            L.sfa_plan_destroy(h)
    assert 43.66 < cap < 43.68


def test_head_group_call_validation_happens_before_any_launch(L):
    """sfa_attention_groups rejects bad arguments without touching the GPU (this runs on CPU)."""
    p = Plan(1, 2, 64, 4, 48, 1)
    S = p.seq
    t = _lib.Tensor(4096, S * 4 * 64, 4 * 64, 64)         # 2 groups of 2 heads
    per = p.info["workspace_bytes"]
    ws = ctypes.c_void_p(1 << 20)
    streams = (ctypes.c_void_p * 2)(None, None)
    G = L.sfa_attention_groups
    assert G(p.handle, 0, t, t, t, t, ws, 2 * per, None, streams, 2) == _lib.SFA_ERR_INVALID
    assert G(p.handle, 2, t, t, t, t, ws, 2 * per - 1, None, streams, 2) == _lib.SFA_ERR_INVALID
    assert G(p.handle, 2, t, t, t, t, None, 2 * per, None, streams, 2) == _lib.SFA_ERR_INVALID
    assert G(p.handle, 2, t, t, t, t, ws, 2 * per, None, None, 2) == _lib.SFA_ERR_INVALID
    assert G(p.handle, 2, t, t, t, t, ws, 2 * per, None, streams, -1) == _lib.SFA_ERR_INVALID
    assert G(None, 2, t, t, t, t, ws, 2 * per, None, streams, 2) == _lib.SFA_ERR_INVALID
    mis = ctypes.c_void_p((1 << 20) + 16)
    assert G(p.handle, 2, t, t, t, t, mis, 2 * per, None, streams, 2) == \
        _lib.SFA_ERR_UNSUPPORTED


@pytest.mark.parametrize("F,T,w", [(4, 48, 1), (8, 208, 2), (3, 80, 5), (13, 32, 2), (0, 16, 0),
                                   (6, 16, 1), (2, 400, 1)])
def test_generic_blocks_match_the_oracle_mask(L, F, T, w):
    """Ablation plan: every (pass, 256-row block, 128-key block) is classified exactly as the
    oracle's mask says (window keys in pass 0, reference keys in pass 1), padding masked."""
    from sparse_attention_frame_amd.api import GenericPlan

    g = GenericPlan(1, 1, 64, F, T, w)
    S = (F + 1) * T
    mask = oracle.mask_matrix(F, T, w)
    frame = np.arange(S) // T
    info = g.info
    assert info["query_blocks"] == -(-S // 256) and info["key_blocks"] == -(-S // 128)
    full = partial = 0
    for p in (0, 1):
        pm = mask & ((frame[None, :] == 0) if p == 1 else (frame[None, :] >= 1))
        for qb in range(info["query_blocks"]):
            rows = slice(qb * 256, min(S, qb * 256 + 256))
            for kb in range(info["key_blocks"]):
                c0, c1 = kb * 128, min(S, kb * 128 + 128)
                sub = pm[rows, c0:c1]
                if not sub.any():
                    want = 0
                elif sub.all() and c1 - c0 == 128:
                    want = 1
                else:
                    want = 2
                assert g.block_class(p, qb, kb) == want, (p, qb, kb)
                full += want == 1
                partial += want == 2
    assert (info["full_blocks"], info["partial_blocks"]) == (full, partial)
    # the two passes cover the mask exactly once
    assert not (mask & (frame[None, :] == 0) & (frame[None, :] >= 1)).any()


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), _lib.SFA_ERR_UNSUPPORTED),
    (dict(model_dim=100), _lib.SFA_ERR_UNSUPPORTED),
    (dict(heads=3, head_dim=64), _lib.SFA_ERR_UNSUPPORTED),      # H*d not a multiple of 256
    (dict(eps=-1.0), _lib.SFA_ERR_INVALID),
    (dict(eps=float("nan")), _lib.SFA_ERR_INVALID),
    (dict(batch=0), _lib.SFA_ERR_INVALID),
    (dict(seq=0), _lib.SFA_ERR_INVALID),
    (dict(heads=0), _lib.SFA_ERR_INVALID),
    (dict(heads=128, head_dim=128, model_dim=65536), _lib.SFA_ERR_UNSUPPORTED),  # W' > 2 GiB
    (dict(batch=4096, seq=262144, heads=512, head_dim=128, model_dim=64),
     _lib.SFA_ERR_UNSUPPORTED),                                   # >= 2^31 workgroup tiles
])
def test_prologue_geometry_errors(L, kw, status):
    """Geometry is checked first, before any pointer is looked at (this runs on CPU)."""
    base = dict(batch=1, seq=100, model_dim=256, heads=4, head_dim=64, eps=1e-6)
    base.update(kw)
    g = _lib.PrologueGeometry(base["batch"], base["seq"], base["model_dim"], base["heads"],
                              base["head_dim"], base["eps"])
    t = _lib.Tensor(1 << 20, 1 << 16, 256, 0)
    P = ctypes.c_void_p
    assert L.sfa_qkv_prologue(ctypes.byref(g), t, P(1 << 22), P(1 << 23), P(1 << 24), t, t, t,
                              None) == status
    assert L.sfa_qkv_prologue(None, t, P(1 << 22), P(1 << 23), P(1 << 24), t, t, t, None) == \
        _lib.SFA_ERR_INVALID


def test_prologue_call_validation_happens_before_any_launch(L):
    """sfa_prologue_fold / sfa_qkv_prologue reject bad arguments without touching the GPU."""
    P = ctypes.c_void_p
    fold = L.sfa_prologue_fold
    assert fold(None, P(4096), P(8192), 16, 64, None) == _lib.SFA_ERR_INVALID
    assert fold(P(4096), P(8192), P(1 << 20), 0, 64, None) == _lib.SFA_ERR_INVALID
    assert fold(P(4096), P(8192), P(1 << 20), 16, 63, None) == _lib.SFA_ERR_UNSUPPORTED
    assert fold(P(4096 + 2), P(8192), P(1 << 20), 16, 64, None) == _lib.SFA_ERR_UNSUPPORTED

    B, S, C, H, d = 1, 100, 256, 4, 64
    g = ctypes.byref(_lib.PrologueGeometry(B, S, C, H, d, 1e-6))
    x = _lib.Tensor(1 << 20, S * C, C, 0)
    w, cs, sn = P(1 << 22), P(1 << 23), P(1 << 24)
    outs = [_lib.Tensor((1 << 26) * (i + 1), S * H * d, H * d, d) for i in range(3)]
    Q = L.sfa_qkv_prologue
    assert Q(g, x, None, cs, sn, *outs, None) == _lib.SFA_ERR_INVALID
    assert Q(g, x, w, None, sn, *outs, None) == _lib.SFA_ERR_INVALID
    assert Q(g, x, w, cs, None, *outs, None) == _lib.SFA_ERR_INVALID
    assert Q(g, _lib.Tensor(None, S * C, C, 0), w, cs, sn, *outs, None) == _lib.SFA_ERR_INVALID
    assert Q(g, x, P((1 << 22) + 8), cs, sn, *outs, None) == _lib.SFA_ERR_UNSUPPORTED
    assert Q(g, x, w, P((1 << 23) + 4), sn, *outs, None) == _lib.SFA_ERR_UNSUPPORTED
    assert Q(g, _lib.Tensor(1 << 20, S * C, C - 8, 0), w, cs, sn, *outs, None) == \
        _lib.SFA_ERR_INVALID                                      # rows overlap
    assert Q(g, _lib.Tensor(1 << 20, S * C, C + 4, 0), w, cs, sn, *outs, None) == \
        _lib.SFA_ERR_UNSUPPORTED                                  # row stride not 16-byte
    bad_out = _lib.Tensor(1 << 26, S * H * d, H * d + 2, d)
    assert Q(g, x, w, cs, sn, bad_out, outs[1], outs[2], None) == _lib.SFA_ERR_UNSUPPORTED
    null_out = _lib.Tensor(None, S * H * d, H * d, d)
    assert Q(g, x, w, cs, sn, outs[0], null_out, outs[2], None) == _lib.SFA_ERR_INVALID
    on_x = _lib.Tensor((1 << 20) + 64, S * H * d, H * d, d)       # output aliasing x
    assert Q(g, x, w, cs, sn, outs[0], on_x, outs[2], None) == _lib.SFA_ERR_INVALID


def test_binding_rejects_host_tensors():
    """The binding refuses host tensors before anything reaches the library (a host pointer
    handed to a kernel would fault the device)."""
    torch = pytest.importorskip("torch")
    import sparse_attention_frame_amd as sfa

    w = torch.zeros(3 * 2 * 128, 64, dtype=torch.bfloat16)
    gamma = torch.ones(64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        sfa.prologue_fold(w, gamma)
    x = torch.zeros(1, 16, 64, dtype=torch.bfloat16)
    cos, sin = torch.zeros(16, 64), torch.zeros(16, 64)
    with pytest.raises(TypeError):
        sfa.qkv_prologue(x, w, cos, sin, 2, 128)
    plan = sfa.Plan(1, 2, 64, 0, 16, 0)
    q = torch.zeros(1, 16, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        sfa.attention(plan, q, q, q)
