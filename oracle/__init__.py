"""CPU oracle for the ZHA decode path: test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The HIP library never uses it.
"""
from . import zha_oracle  # noqa: F401
