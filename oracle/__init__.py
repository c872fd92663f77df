"""fp64 CPU oracle for the sign-binarised linear layers (OneBit, DBF).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg use it.  It shares no code, constant or
helper with the HIP library under ``bit_weight_linear_amd/``.

The oracle is NumPy in float64.  Every function cites the passage of the pages
it follows.  Parity status of each function is stated in ``reference.py``.
"""
from .reference import *  # noqa: F401,F403
