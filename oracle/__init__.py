"""fp64 CPU oracle for the Star Attention hot path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.
"""
from . import star_oracle  # noqa: F401
