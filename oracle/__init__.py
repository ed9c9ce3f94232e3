"""CPU oracle for frame-aligned window-sparse attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package. The HIP library and its
Python binding never do, and this package never imports them: the two
implementations share no code, tables or helpers.

Source: "HeyGen x Google Cloud: Bringing Avatar IV to TPUs" (Google Developers
Blog), sections "Deleting the mask" (Fig. 3), "Unchaining softmax" (Fig. 4)
and "Proving pixels unchanged".

What it computes, in float64:

* ``attention`` -- dense softmax attention with the frame-window mask applied
  as -inf logits: the plain definition that the single-pass, no-predicate
  kernel reaches exactly (blocks are either entirely inside the mask or
  entirely skipped, and the reference frame's blocks are ordinary blocks of
  the same softmax); ``attention_block`` is its unit of work, a block of rows
  of one (batch, head) inside one query frame, which the full-size tests run
  over a thread pool.
* ``head_stats`` -- per (batch, head): the key mean, the largest mean-centred
  key norm, the largest query norm, the Cauchy-Schwarz bound and the
  eligibility flag for the fixed-maximum path.
* ``row_offsets`` -- the per-row fixed maximum used by the fixed-max path
  (a diagnostic: the output does not depend on it in exact arithmetic).
* ``frame_stats`` / ``frame_row_offsets`` -- the same bound taken per
  (batch, head, query frame): the largest centred key norm over the frames a
  query frame can see, and per-query-frame eligibility.
* ``brute.attention_brute`` -- pure-Python loops over explicitly enumerated
  visible key sets (tiny inputs only).
* ``prologue.qkv_prologue`` -- the attention's input chain (section "Layout as
  ABI"): RMSNorm, the q/k/v projection, rotary embedding of q and k, head
  packing; ``prologue.rms_norm`` and ``prologue.rotate_pairs`` are its steps.

Pins (``tests/test_oracle.py``, all CPU): brute force, torch's fp64
scaled-dot-product attention with an independently built mask, closed-form
frame-pair counts, exact-value constructions for the bound (including the
inclusive threshold and a zero-gap row), and the invariants (key centring,
bound >= row max, full window == dense attention, q = 0 gives window means,
frame-indicator values give zero mass outside the window, permutation inside a
frame). No function here is "parity unpinned".
"""
from .attention import (  # noqa: F401
    attention,
    attention_block,
    attention_rows,
    frame_row_offsets,
    frame_stats,
    head_stats,
    key_frames,
    mask_matrix,
    row_offsets,
)
from .brute import attention_brute  # noqa: F401
from .prologue import qkv_prologue, rms_norm, rotate_pairs  # noqa: F401
