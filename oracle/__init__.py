"""CPU oracle of the FMDQ differential linear layer (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may use this package.  See ``oracle/fmdq.py``.
"""
from . import fmdq  # noqa: F401
