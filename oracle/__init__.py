"""fp64 CPU oracle of the Gated DeltaNet layer core.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check in
``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py``; never by the
product package, which shares no code with it.
"""
from .oracle import *  # noqa: F401,F403
