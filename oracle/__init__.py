"""fp64 CPU oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library.
"""
from .pa_oracle import (append, attend, attend_partitioned, attend_workload,  # noqa: F401
                        bad_entries, half_to_double, max_threads)
