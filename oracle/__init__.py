"""CPU oracle of the ResidualKV cache-write path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package; the GPU library never does.
"""
from . import rkv_oracle  # noqa: F401
