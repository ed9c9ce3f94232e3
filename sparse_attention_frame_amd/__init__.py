"""Frame-aligned window-sparse attention on MI355X (gfx950).

The computation lives in libsfa.so (hand-written HIP kernels behind the C ABI
of include/sfa.h); this package only loads it and marshals torch tensors.
Importing the package does not need a GPU; calling the kernels does, and
raises if the library was not built.
"""
from ._lib import SfaError, lib  # noqa: F401
from .api import (  # noqa: F401
    GenericPlan,
    Plan,
    attention,
    attention_groups,
    attention_static,
    frame_stats,
    fwd,
    generic_attention,
    head_stats,
    norms,
    prologue_fold,
    qkv_prologue,
    row_norms,
    sfa_attention,
    sfa_attention_groups,
    sfa_attention_static,
    sfa_fwd,
    sfa_generic_attention,
    sfa_norms,
    sfa_prologue_fold,
    sfa_qkv_prologue,
    sfa_read_frame_stats,
    sfa_read_head_stats,
    sfa_read_row_norms,
    sfa_read_staged,
    staged,
)
