"""fp64 CPU oracle for exact tiled masked softmax attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table
or constant with the HIP library (``exact_tiled_softmax_amd``); both receive
their inputs from the seeded generators in ``workloads``, which hold none of
the method's arithmetic.

Modules
  dense    masked softmax attention (the plain dense definition) and its
           analytic vector-Jacobian product, with optional inverted dropout.
  summary  the block-summary recurrence (m, l, z) with the empty state, used
           to reproduce the intermediate summaries the pages print.
  sparse   shared-KV top-k sparse attention with an attention sink, forward
           and backward, including the tied K/V row merge.
  philox   Philox4x32-10 written from Salmon et al., "Parallel random numbers:
           as easy as 1, 2, 3" (SC'11), and the dropout keep mask built on it.
  fd       central finite differences used to pin the analytic VJPs.

Every function is plain NumPy in float64 and states the passage it follows.
"""

from . import dense, fd, philox, sparse, summary  # noqa: F401
