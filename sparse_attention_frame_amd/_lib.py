"""ctypes loader for libsfa.so (argument marshalling only; all compute is in the HIP library)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# SFA_LIBRARY names another build of the same library (the sanitizer build of the host
# code that the CPU tests load); by default the in-tree libsfa.so
LIB_PATH = os.environ.get("SFA_LIBRARY") or os.path.join(_HERE, "libsfa.so")

SFA_OK = 0
SFA_ERR_INVALID = -1
SFA_ERR_UNSUPPORTED = -2
SFA_ERR_HIP = -3
SFA_ERR_NOMEM = -4
SFA_ERR_TOO_LARGE = -5


class Geometry(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("frames", ctypes.c_int32),
                ("tokens_per_frame", ctypes.c_int32), ("window", ctypes.c_int32),
                ("scale", ctypes.c_float), ("bound_limit", ctypes.c_float)]


class Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_s", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class PlanOptions(ctypes.Structure):
    _fields_ = [("block_q", ctypes.c_int32), ("waves_per_item", ctypes.c_int32),
                ("lds_stages", ctypes.c_int32), ("bound_mode", ctypes.c_int32),
                ("key_split", ctypes.c_int32), ("wave_rows", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("block_q", ctypes.c_int32), ("granule", ctypes.c_int32),
                ("waves_per_item", ctypes.c_int32), ("items", ctypes.c_int32),
                ("active_pairs", ctypes.c_int64), ("active_flops", ctypes.c_double),
                ("io_bytes", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t),
                ("bound_mode", ctypes.c_int32), ("split_frames", ctypes.c_int32),
                ("wave_rows", ctypes.c_int32)]


class GenericInfo(ctypes.Structure):
    _fields_ = [("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("query_blocks", ctypes.c_int32), ("key_blocks", ctypes.c_int32),
                ("full_blocks", ctypes.c_int64), ("partial_blocks", ctypes.c_int64),
                ("computed_pairs", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t)]


class PrologueGeometry(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq", ctypes.c_int32),
                ("model_dim", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("eps", ctypes.c_float)]


# every symbol include/sfa.h declares
EXPORTS = (
    "sfa_plan_create", "sfa_plan_create_ex", "sfa_plan_destroy", "sfa_plan_get_info",
    "sfa_plan_key_ranges", "sfa_plan_item", "sfa_plan_item_keys", "sfa_norms", "sfa_fwd", "sfa_attention",
    "sfa_attention_static",
    "sfa_attention_groups", "sfa_read_head_stats", "sfa_read_row_norms", "sfa_read_frame_stats",
    "sfa_read_staged",
    "sfa_prologue_fold", "sfa_qkv_prologue",
    "sfa_generic_create", "sfa_generic_destroy", "sfa_generic_get_info", "sfa_generic_block_class",
    "sfa_generic_attention", "sfa_status_str",
)

_lib = None


class SfaError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = _lib.sfa_status_str(status).decode() if _lib is not None else str(status)
        super().__init__(f"{what}: {msg} (status {status})")
        self.status = status


def _declare(lib):
    P = ctypes.c_void_p
    i32p = ctypes.POINTER(ctypes.c_int32)
    f32p = ctypes.POINTER(ctypes.c_float)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    sigs = {
        "sfa_plan_create": (ctypes.c_int, [ctypes.POINTER(Geometry), ctypes.POINTER(P)]),
        "sfa_plan_create_ex": (ctypes.c_int, [ctypes.POINTER(Geometry),
                                              ctypes.POINTER(PlanOptions), ctypes.POINTER(P)]),
        "sfa_plan_destroy": (None, [P]),
        "sfa_plan_get_info": (ctypes.c_int, [P, ctypes.POINTER(PlanInfo)]),
        "sfa_plan_key_ranges": (ctypes.c_int, [P, ctypes.c_int32, i32p, i32p]),
        "sfa_plan_item": (ctypes.c_int, [P, ctypes.c_int32, i32p]),
        "sfa_plan_item_keys": (ctypes.c_int, [P, ctypes.c_int32, i32p, i32p, i32p]),
        "sfa_norms": (ctypes.c_int, [P, Tensor, Tensor, Tensor, P, ctypes.c_size_t, P]),
        "sfa_fwd": (ctypes.c_int, [P, Tensor, Tensor, Tensor, Tensor, P, ctypes.c_size_t, P]),
        "sfa_attention": (ctypes.c_int, [P, Tensor, Tensor, Tensor, Tensor, P, ctypes.c_size_t,
                                         P]),
        "sfa_attention_static": (ctypes.c_int, [P, Tensor, Tensor, Tensor, Tensor, P]),
        "sfa_attention_groups": (ctypes.c_int, [P, ctypes.c_int32, Tensor, Tensor, Tensor, Tensor,
                                                P, ctypes.c_size_t, P, ctypes.POINTER(P),
                                                ctypes.c_int32]),
        "sfa_read_head_stats": (ctypes.c_int, [P, P, ctypes.c_size_t, f32p, f32p, f32p, f32p,
                                               u8p, P]),
        "sfa_read_row_norms": (ctypes.c_int, [P, P, ctypes.c_size_t, f32p, f32p, P]),
        "sfa_read_frame_stats": (ctypes.c_int, [P, P, ctypes.c_size_t, f32p, f32p, u8p, P]),
        "sfa_read_staged": (ctypes.c_int, [P, P, ctypes.c_size_t, ctypes.POINTER(ctypes.c_uint16),
                                           ctypes.POINTER(ctypes.c_uint16), P]),
        "sfa_prologue_fold": (ctypes.c_int, [P, P, P, ctypes.c_int32, ctypes.c_int32, P]),
        "sfa_qkv_prologue": (ctypes.c_int, [ctypes.POINTER(PrologueGeometry), Tensor, P, P, P,
                                            Tensor, Tensor, Tensor, P]),
        "sfa_generic_create": (ctypes.c_int, [ctypes.POINTER(Geometry), ctypes.POINTER(P)]),
        "sfa_generic_destroy": (None, [P]),
        "sfa_generic_get_info": (ctypes.c_int, [P, ctypes.POINTER(GenericInfo)]),
        "sfa_generic_block_class": (ctypes.c_int, [P, ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.c_int32, i32p]),
        "sfa_generic_attention": (ctypes.c_int, [P, Tensor, Tensor, Tensor, Tensor, P,
                                                 ctypes.c_size_t, P]),
        "sfa_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def lib():
    """Load libsfa.so once. Raises ImportError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m sparse_attention_frame_amd.build, or __graft_entry__.build())")
        # torch ships its own libamdhip64; load it first so the library binds to the
        # same HIP runtime as torch's streams and allocations
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        _lib = ctypes.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


def check(status: int, what: str):
    if status != SFA_OK:
        raise SfaError(status, what)
