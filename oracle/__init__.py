"""fp64 CPU oracle of the Llama decoder-layer forward (test infrastructure only).

Only tests/, ``__graft_entry__.smoke()`` and bench.py's ``cpu_baseline`` leg may
import this package; the GPU library neither imports nor calls it.
"""
from . import ref, brute  # noqa: F401
