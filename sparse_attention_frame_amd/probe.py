"""ctypes binding of libsfa_probe.so: the matrix-core microbenchmarks (include/sfa_probe.h)
that the benchmark reports the attention kernel against. Marshalling only."""
from __future__ import annotations

import ctypes
import os

from . import _lib as L

PROBE_LIB_PATH = os.path.join(L._HERE, "libsfa_probe.so")

MFMA_CHAIN = 0      # independent v_mfma_f32_32x32x16_bf16 chains, no memory
TILE_LOOP = 1       # attention tile loop, 32 query rows per wave, operands from LDS
TILE_LOOP64 = 2     # the same with 64 query rows per wave
TILE_NOEXP = 3      # the 32-row tile loop without the softmax

EXPORTS = ("sfa_probe_scratch_bytes", "sfa_probe_run")


class Result(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double), ("tflops", ctypes.c_double),
                ("clock_ghz", ctypes.c_double), ("mfma_busy", ctypes.c_double)]


_plib = None


def lib():
    global _plib
    if _plib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise ImportError(f"{PROBE_LIB_PATH} is missing: build the HIP libraries first")
        L.lib()   # binds torch's HIP runtime first
        _plib = ctypes.CDLL(PROBE_LIB_PATH)
        _plib.sfa_probe_scratch_bytes.restype = ctypes.c_size_t
        _plib.sfa_probe_scratch_bytes.argtypes = []
        _plib.sfa_probe_run.restype = ctypes.c_int
        _plib.sfa_probe_run.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                        ctypes.POINTER(Result)]
    return _plib


def run(kind: int, waves: int = 8, iters: int = 20000, stream=None, scratch=None) -> dict:
    """One timed launch (after a short warm-up launch) on the current device."""
    import torch

    pl = lib()
    nbytes = pl.sfa_probe_scratch_bytes()
    if scratch is None:
        scratch = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    if stream is None:
        stream = torch.cuda.current_stream()
    r = Result()
    st = pl.sfa_probe_run(kind, waves, iters, ctypes.c_void_p(scratch.data_ptr()),
                          scratch.numel(), ctypes.c_void_p(stream.cuda_stream), ctypes.byref(r))
    if st != 0:
        raise RuntimeError(f"sfa_probe_run(kind={kind}, waves={waves}) failed with status {st}")
    return {"ms": r.ms, "tflops": r.tflops, "clock_ghz": r.clock_ghz, "mfma_busy": r.mfma_busy}
