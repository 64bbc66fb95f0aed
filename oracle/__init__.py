"""fp64 CPU oracle for MLA paged decode (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  The HIP library never imports it.
"""
from .mla_oracle import *  # noqa: F401,F403
