"""FP64 CPU oracle for the Gated DeltaNet-2 (GDN-2) forward recurrence.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call, link
or execute anything in this package; only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.

Two implementations of the *same* definition live here and are pinned by the
same tests:

* :mod:`oracle.recurrence` -- numpy, vectorised over value heads only.
* :mod:`oracle.c_oracle` -- a plain C loop nest (``gdn2_oracle.c``) reached
  through ctypes, for full-size workloads. It is compiled by
  :func:`oracle.build.build_c_oracle`.

Both follow the recurrence printed in the FlashInfer
``chunk_gated_delta_rule2`` documentation (recurrence display equation), token
by token, with no chunking, in float64.

The backward pass (gradients of every input and of the initial state) has the
same two forms: :mod:`oracle.recurrence_bwd` (numpy) and ``gdn2_oracle_bwd``
in the same C file (reached through :func:`oracle.c_oracle.gdn2_recurrence_bwd_c`),
both the reverse sweep of the chain rule through the token recurrence, pinned
by ``tests/test_oracle_bwd_pins.py``.
"""

from .recurrence import gdn2_recurrence, gdn2_sequence, resolve_scale
from .recurrence_bwd import gdn2_recurrence_bwd

__all__ = ["gdn2_recurrence", "gdn2_sequence", "resolve_scale", "gdn2_recurrence_bwd"]
