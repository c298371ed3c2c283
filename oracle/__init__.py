"""CPU oracle for MoE expert-parallel dispatch layout, dispatch and combine.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
statement of what the GPU path computes.  Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py`` may import
it.  It shares no code with the HIP library under
``combine_get_dispatch_07_amd/`` and never imports it; the product path never
routes through it.

Modules
-------
``numerics``   bf16 and OCP FP8 E4M3 codecs, from their definitions.
``moe_oracle`` vectorised numpy oracle for every step (all workload sizes).
``bruteforce`` pure-Python loop oracle for tiny inputs (an independent pin).

Every function in ``moe_oracle`` is pinned by ``tests/test_oracle_pins.py``
against hand-worked golden cases, closed forms, invariants, library routines
(torch's bf16 and float8_e4m3fn conversions) and the brute-force loops.
"""
from . import numerics, moe_oracle, bruteforce  # noqa: F401
