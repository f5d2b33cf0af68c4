"""CPU oracle for the DSA hot path (test infrastructure only).

Only tests, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
may import this package.  It shares no code with the HIP library.
"""
from .dsa_oracle import *  # noqa: F401,F403
