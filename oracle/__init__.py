"""CPU oracle for the packed 4-direction 2D MDLSTM layer.

TEST INFRASTRUCTURE ONLY. Plain, slow, float64 NumPy code written from the
pages ("No Padding Please: Efficient Neural Handwriting Recognition", and the
RETURNN paper's MDLSTM description in §4.2). Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. It shares no code with the HIP library and never imports it; the
only module both sides use is ``workloads`` (seeded inputs, no arithmetic of
the method).

Modules:
  pack       example packing (§IX-B (packing algorithm details, Algorithm 1)) and the padded stack
  canvas     scatter onto the canvas, direction sum and un-packing (§V-A)
  mdlstm     the cell, forward and 2D BPTT, per-cell and per-diagonal forms
  leaky      the Leaky-LP cell (lambda gate, two output gates), forward and 2D BPTT (§III, Fig. 4(b), §IX-A)
  blockconv  block-strided convolution with tensor-list chunking (§V-B)
  stack      three MDLSTM levels with block convs, re-packed per level (§II, §V)

Every function is pinned by a ``-m "not gpu"`` test in ``tests/test_oracle_*.py``
against something other than itself (brute force, closed forms, a library
routine, finite differences, invariants the pages state).
"""

from . import pack, canvas, mdlstm, leaky, blockconv, stack  # noqa: F401
