"""CPU oracle of the Sparse Delta Memory layer forward (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package. The HIP path never calls it, and it never calls the HIP path.
"""
from .sdm_oracle import *  # noqa: F401,F403
