"""CPU oracle for training-free block-sparse attention over a 3D video token grid.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package. The product path (the HIP library under
``block_sparse_attention_bsa_amd`` and its binding) never imports it, and this package imports
nothing from the product path: the two share no code. Both consume the same seeded inputs from
``gen``.

Every function is a plain, slow, fp64 restatement of what the pages define; see
``oracle.bsa_oracle`` for the per-function citations. Parity status: every function is pinned by
tests under ``tests/test_oracle_*.py`` (invariants, closed forms, brute force, library routines,
finite differences) except the readings listed as "parity unpinned" in the module docstring.
"""
from .bsa_oracle import *  # noqa: F401,F403
