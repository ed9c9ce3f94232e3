"""Python face of the C ABI in include/sfa.h (same names; marshalling only).

Tensors are torch.bfloat16 device tensors shaped [B, S, H, d] with the last
dimension contiguous; any batch/token/head strides (multiples of 8 elements)
are passed through, so BHSD storage or a head-subset view works unchanged.
torch supplies device memory and the stream; every step of the computation
runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _lib
from ._lib import (GenericInfo, Geometry, PlanInfo, PlanOptions, PrologueGeometry, Tensor,
                   check, lib)


def _stream_ptr(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Plan:
    """sfa_plan_create: geometry -> tiles and the largest-first work-item order."""

    def __init__(self, batch: int, heads: int, head_dim: int, frames: int,
                 tokens_per_frame: int, window: int, scale: float = 0.0,
                 bound_limit: float = 40.0, block_q: int = 0, waves: int = 0,
                 lds_stages: int = 0, bound_mode: int = 0, key_split: int = 0,
                 wave_rows: int = 0):
        self.geometry = Geometry(batch, heads, head_dim, frames, tokens_per_frame, window,
                                 scale, bound_limit)
        handle = ctypes.c_void_p()
        L = lib()
        if block_q or waves or lds_stages or bound_mode or key_split or wave_rows:
            opts = PlanOptions(block_q, waves, lds_stages, bound_mode, key_split, wave_rows)
            st = L.sfa_plan_create_ex(ctypes.byref(self.geometry), ctypes.byref(opts),
                                      ctypes.byref(handle))
        else:
            st = L.sfa_plan_create(ctypes.byref(self.geometry), ctypes.byref(handle))
        check(st, "sfa_plan_create")
        self._h = handle
        info = PlanInfo()
        check(L.sfa_plan_get_info(self._h, ctypes.byref(info)), "sfa_plan_get_info")
        self.info = {name: getattr(info, name) for name, _ in PlanInfo._fields_}
        self.seq = (frames + 1) * tokens_per_frame

    @classmethod
    def for_workload(cls, wl, **kw):
        return cls(wl.batch, wl.heads, wl.head_dim, wl.frames, wl.tokens_per_frame, wl.window,
                   **kw)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib._lib is not None:
            _lib._lib.sfa_plan_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def key_ranges(self, frame: int):
        r = (ctypes.c_int32 * 4)()
        n = ctypes.c_int32()
        check(lib().sfa_plan_key_ranges(self._h, frame, r, ctypes.byref(n)),
              "sfa_plan_key_ranges")
        return [(r[2 * i], r[2 * i + 1]) for i in range(n.value)]

    def item(self, index: int):
        out = (ctypes.c_int32 * 4)()
        check(lib().sfa_plan_item(self._h, index, out), "sfa_plan_item")
        return tuple(out)

    def item_keys(self, index: int):
        """(half, [(start, end), ...]): half -1 for a whole item, 0 / 1 for a key half."""
        half = ctypes.c_int32()
        r = (ctypes.c_int32 * 4)()
        n = ctypes.c_int32()
        check(lib().sfa_plan_item_keys(self._h, index, ctypes.byref(half), r, ctypes.byref(n)),
              "sfa_plan_item_keys")
        return half.value, [(r[2 * i], r[2 * i + 1]) for i in range(n.value)]

    def workspace(self, device=None):
        import torch

        return torch.empty(self.info["workspace_bytes"], dtype=torch.uint8,
                           device=device or "cuda")


def as_tensor(t, plan: Plan, name: str) -> Tensor:
    import torch

    g = plan.geometry
    shape = (g.batch, plan.seq, g.heads, g.head_dim)
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be torch.bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if tuple(t.shape) != shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, plan expects {shape}")
    if t.stride(3) != 1:
        raise ValueError(f"{name} needs a contiguous head dimension")
    return Tensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _ws(plan, workspace, device):
    if workspace is None:
        workspace = plan.workspace(device)
    return workspace


def _ws_args(ws):
    """(pointer, size in bytes) of a workspace tensor, which must be a device tensor."""
    if not ws.is_cuda:
        raise TypeError("the workspace must be a device tensor")
    if not ws.is_contiguous():
        raise ValueError("the workspace must be contiguous")
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


def sfa_norms(plan: Plan, q, k, v, workspace=None, stream=None):
    """Prologue: norm array (from q, k) and V^T staging (from v) into the workspace."""
    ws = _ws(plan, workspace, q.device)
    check(lib().sfa_norms(plan.handle, as_tensor(q, plan, "q"), as_tensor(k, plan, "k"),
                          as_tensor(v, plan, "v"), *_ws_args(ws),
                          _stream_ptr(stream)), "sfa_norms")
    return ws


def sfa_fwd(plan: Plan, q, k, v, out=None, workspace=None, stream=None):
    import torch

    if workspace is None:
        raise ValueError("sfa_fwd needs the workspace filled by sfa_norms")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    check(lib().sfa_fwd(plan.handle, as_tensor(q, plan, "q"), as_tensor(k, plan, "k"),
                        as_tensor(v, plan, "v"), as_tensor(out, plan, "o"),
                        *_ws_args(workspace),
                        _stream_ptr(stream)), "sfa_fwd")
    return out


def sfa_attention(plan: Plan, q, k, v, out=None, workspace=None, stream=None):
    """sfa_norms + sfa_fwd on one stream. Returns (out, workspace)."""
    import torch

    ws = _ws(plan, workspace, q.device)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    check(lib().sfa_attention(plan.handle, as_tensor(q, plan, "q"), as_tensor(k, plan, "k"),
                              as_tensor(v, plan, "v"), as_tensor(out, plan, "o"),
                              *_ws_args(ws), _stream_ptr(stream)),
          "sfa_attention")
    return out, ws


def sfa_attention_static(plan: Plan, q, k, v, out=None, stream=None):
    """sfa_attention on the library's fixed per-GPU workspace (no workspace argument, no
    device allocation by the library; plans beyond its 64 MiB raise). Returns out."""
    import torch

    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    check(lib().sfa_attention_static(plan.handle, as_tensor(q, plan, "q"),
                                     as_tensor(k, plan, "k"), as_tensor(v, plan, "v"),
                                     as_tensor(out, plan, "o"), _stream_ptr(stream)),
          "sfa_attention_static")
    return out


def sfa_attention_groups(group_plan: Plan, groups: int, q, k, v, out=None, workspace=None,
                         streams=(), stream=None):
    """sfa_attention on `groups` consecutive head groups of q, k, v ([B, S, groups*Hg, d]),
    group g on streams[g % len(streams)] (or on `stream` when streams is empty), each with
    its own slice of the workspace. Returns (out, workspace)."""
    import torch

    g = group_plan.geometry
    shape = (g.batch, group_plan.seq, groups * g.heads, g.head_dim)
    for name, t in (("q", q), ("k", k), ("v", v)) + ((("o", out),) if out is not None else ()):
        if t.dtype != torch.bfloat16 or not t.is_cuda or tuple(t.shape) != shape or \
                t.stride(3) != 1:
            raise ValueError(f"{name} must be a bf16 device tensor {shape} with contiguous d")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if workspace is None:
        workspace = torch.empty(groups * group_plan.info["workspace_bytes"], dtype=torch.uint8,
                                device=q.device)
    ts = [Tensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2)) for t in (q, k, v, out)]
    arr = (ctypes.c_void_p * max(1, len(streams)))(*[s.cuda_stream for s in streams])
    check(lib().sfa_attention_groups(group_plan.handle, groups, *ts,
                                     *_ws_args(workspace),
                                     _stream_ptr(stream), arr, len(streams)),
          "sfa_attention_groups")
    return out, workspace


def sfa_read_head_stats(plan: Plan, workspace, stream=None):
    g = plan.geometry
    bh = g.batch * g.heads
    mu = np.empty((g.batch, g.heads, g.head_dim), np.float32)
    kmax = np.empty((g.batch, g.heads), np.float32)
    qmax = np.empty((g.batch, g.heads), np.float32)
    bound = np.empty((g.batch, g.heads), np.float32)
    elig = np.empty((g.batch, g.heads), np.uint8)
    f = ctypes.POINTER(ctypes.c_float)
    check(lib().sfa_read_head_stats(plan.handle, *_ws_args(workspace),
                                    mu.ctypes.data_as(f), kmax.ctypes.data_as(f),
                                    qmax.ctypes.data_as(f), bound.ctypes.data_as(f),
                                    elig.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                                    _stream_ptr(stream)), "sfa_read_head_stats")
    assert bh == kmax.size
    return {"mu": mu, "kmax": kmax, "qmax": qmax, "bound": bound, "eligible": elig.astype(bool)}


def sfa_read_row_norms(plan: Plan, workspace, stream=None):
    g = plan.geometry
    qn = np.empty((g.batch, g.heads, plan.seq), np.float32)
    qmu = np.empty((g.batch, g.heads, plan.seq), np.float32)
    f = ctypes.POINTER(ctypes.c_float)
    check(lib().sfa_read_row_norms(plan.handle, *_ws_args(workspace),
                                   qn.ctypes.data_as(f), qmu.ctypes.data_as(f),
                                   _stream_ptr(stream)), "sfa_read_row_norms")
    return qn, qmu


def sfa_read_frame_stats(plan: Plan, workspace, stream=None):
    """Per (batch, head, query frame): kvis, bound and eligible, arrays [B, H, F + 1]."""
    g = plan.geometry
    shape = (g.batch, g.heads, g.frames + 1)
    kvis = np.empty(shape, np.float32)
    bound = np.empty(shape, np.float32)
    elig = np.empty(shape, np.uint8)
    f = ctypes.POINTER(ctypes.c_float)
    check(lib().sfa_read_frame_stats(plan.handle, *_ws_args(workspace),
                                     kvis.ctypes.data_as(f), bound.ctypes.data_as(f),
                                     elig.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                                     _stream_ptr(stream)), "sfa_read_frame_stats")
    return {"kvis": kvis, "bound": bound, "eligible": elig.astype(bool)}


def sfa_read_staged(plan: Plan, workspace, stream=None):
    """The staged k and v the attention kernel reads: two uint16 arrays [B, H, S * d] in
    the granule layouts described at sfa_norms (bf16 bit patterns)."""
    g = plan.geometry
    shape = (g.batch, g.heads, plan.seq * g.head_dim)
    kst = np.empty(shape, np.uint16)
    vst = np.empty(shape, np.uint16)
    u16 = ctypes.POINTER(ctypes.c_uint16)
    check(lib().sfa_read_staged(plan.handle, *_ws_args(workspace), kst.ctypes.data_as(u16),
                                vst.ctypes.data_as(u16), _stream_ptr(stream)),
          "sfa_read_staged")
    return kst, vst


def sfa_prologue_fold(w, gamma, stream=None):
    """W' = bf16(gamma * W) for bf16 device tensors W [N, C], gamma [C]."""
    import torch

    if w.dtype != torch.bfloat16 or gamma.dtype != torch.bfloat16 or w.dim() != 2 or \
            not w.is_contiguous() or tuple(gamma.shape) != (w.shape[1],) or \
            not gamma.is_contiguous():
        raise ValueError("w must be a contiguous bf16 [N, C] tensor and gamma a contiguous "
                         "bf16 [C] tensor")
    if not (w.is_cuda and gamma.is_cuda):
        raise TypeError("w and gamma must be device tensors")
    out = torch.empty_like(w)
    check(lib().sfa_prologue_fold(ctypes.c_void_p(w.data_ptr()),
                                  ctypes.c_void_p(gamma.data_ptr()),
                                  ctypes.c_void_p(out.data_ptr()), w.shape[0], w.shape[1],
                                  _stream_ptr(stream)), "sfa_prologue_fold")
    return out


def sfa_qkv_prologue(x, w_folded, cos, sin, heads: int, head_dim: int, eps: float = 1e-6,
                     q=None, k=None, v=None, stream=None):
    """Fused RMSNorm -> projection -> rotary -> head packing. x bf16 [B, S, C] (C
    contiguous), w_folded bf16 [3*H*d, C], cos/sin float32 [S, d/2]. Returns (q, k, v),
    bf16 [B, S, H, d] (or the given output tensors, any strides with d contiguous)."""
    import torch

    B, S, C = x.shape
    if x.dtype != torch.bfloat16 or x.stride(2) != 1:
        raise ValueError("x must be bf16 [B, S, C] with C contiguous")
    for name, t in (("x", x), ("w_folded", w_folded), ("cos", cos), ("sin", sin)) + \
            tuple((n, t) for n, t in (("q", q), ("k", k), ("v", v)) if t is not None):
        if not t.is_cuda:
            raise TypeError(f"{name} must be a device tensor")
    if w_folded.dtype != torch.bfloat16 or tuple(w_folded.shape) != (3 * heads * head_dim, C) \
            or not w_folded.is_contiguous():
        raise ValueError("w_folded must be a contiguous bf16 [3*H*d, C] tensor")
    for t in (cos, sin):
        if t.dtype != torch.float32 or tuple(t.shape) != (S, head_dim // 2) or \
                not t.is_contiguous():
            raise ValueError("cos / sin must be contiguous float32 [S, d/2]")
    g = PrologueGeometry(B, S, C, heads, head_dim, eps)
    outs = []
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t is None:
            t = torch.empty((B, S, heads, head_dim), dtype=torch.bfloat16, device=x.device)
        if t.dtype != torch.bfloat16 or tuple(t.shape) != (B, S, heads, head_dim) or \
                t.stride(3) != 1:
            raise ValueError(f"{name} must be bf16 [B, S, H, d] with d contiguous")
        outs.append(t)
    xt = Tensor(x.data_ptr(), x.stride(0), x.stride(1), 0)
    ts = [Tensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2)) for t in outs]
    check(lib().sfa_qkv_prologue(ctypes.byref(g), xt, ctypes.c_void_p(w_folded.data_ptr()),
                                 ctypes.c_void_p(cos.data_ptr()), ctypes.c_void_p(sin.data_ptr()),
                                 *ts, _stream_ptr(stream)), "sfa_qkv_prologue")
    return tuple(outs)


class GenericPlan:
    """Ablation (sfa_generic_create): generic 256 x 128 block-sparse tiles, element masks on
    partial blocks, window and reference-frame keys as two passes plus a merge."""

    def __init__(self, batch: int, heads: int, head_dim: int, frames: int,
                 tokens_per_frame: int, window: int, scale: float = 0.0):
        self.geometry = Geometry(batch, heads, head_dim, frames, tokens_per_frame, window,
                                 scale, 40.0)
        handle = ctypes.c_void_p()
        check(lib().sfa_generic_create(ctypes.byref(self.geometry), ctypes.byref(handle)),
              "sfa_generic_create")
        self._h = handle
        info = GenericInfo()
        check(lib().sfa_generic_get_info(self._h, ctypes.byref(info)), "sfa_generic_get_info")
        self.info = {name: getattr(info, name) for name, _ in GenericInfo._fields_}
        self.seq = (frames + 1) * tokens_per_frame

    @classmethod
    def for_workload(cls, wl, **kw):
        return cls(wl.batch, wl.heads, wl.head_dim, wl.frames, wl.tokens_per_frame, wl.window,
                   **kw)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib._lib is not None:
            _lib._lib.sfa_generic_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def block_class(self, pass_: int, query_block: int, key_block: int) -> int:
        c = ctypes.c_int32()
        check(lib().sfa_generic_block_class(self._h, pass_, query_block, key_block,
                                            ctypes.byref(c)), "sfa_generic_block_class")
        return c.value

    def workspace(self, device=None):
        import torch

        return torch.empty(self.info["workspace_bytes"], dtype=torch.uint8,
                           device=device or "cuda")


def sfa_generic_attention(plan: GenericPlan, q, k, v, out=None, workspace=None, stream=None):
    """The generic two-pass ablation on one stream. Returns (out, workspace)."""
    import torch

    if workspace is None:
        workspace = plan.workspace(q.device)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    check(lib().sfa_generic_attention(plan.handle, as_tensor(q, plan, "q"),
                                      as_tensor(k, plan, "k"), as_tensor(v, plan, "v"),
                                      as_tensor(out, plan, "o"),
                                      *_ws_args(workspace),
                                      _stream_ptr(stream)), "sfa_generic_attention")
    return out, workspace


# short aliases
norms = sfa_norms
fwd = sfa_fwd
attention = sfa_attention
attention_static = sfa_attention_static
attention_groups = sfa_attention_groups
head_stats = sfa_read_head_stats
row_norms = sfa_read_row_norms
frame_stats = sfa_read_frame_stats
staged = sfa_read_staged
generic_attention = sfa_generic_attention
prologue_fold = sfa_prologue_fold
qkv_prologue = sfa_qkv_prologue
