"""fp64 CPU oracle of the selective-SSM scan -- TEST INFRASTRUCTURE ONLY.

Two independent implementations of one plain definition: ``oracle_c`` (C,
threads over channels) and ``oracle_np`` (NumPy, vectorised over channels).
Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The HIP path never does, and it
shares no code with it.

Every function is pinned in ``tests/test_oracle_*.py`` against closed forms,
identities and brute force.  Parity is pinned for all three functions
(forward, backward, decode).
"""
from . import oracle_c, oracle_np  # noqa: F401
