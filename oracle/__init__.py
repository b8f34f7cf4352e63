"""CPU oracle for the selective-recompute attention core and the SP norm region.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It is plain, slow, float64
numpy that materialises the full score matrix; it shares no code with the HIP
library and never imports it.

Modules:
* ``philox``    -- Philox4x32-10 and the attention / hidden dropout keep-masks
* ``attention`` -- attention core forward and recompute backward
* ``norm``      -- LayerNorm / RMSNorm + dropout + residual, forward and backward
* ``ledger``    -- activation bytes per layer (none / selective / full, TP / SP)

Every function is pinned by ``tests/test_oracle_*.py`` to facts the pages or
the mathematics fix (library routines, closed forms, finite differences,
an independent Philox implementation, the pages' worked example).
"""
from . import philox, attention, norm, ledger  # noqa: F401
