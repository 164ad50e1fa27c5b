"""CPU oracle for the sparse MLA hot path: test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` import this package.  It shares no code with the HIP library.
"""
from . import ref  # noqa: F401
