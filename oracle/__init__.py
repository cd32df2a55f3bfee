"""The oracle: plain float64 CPU attention that the HIP library is checked against.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the package smoke check and the
benchmark's CPU-baseline leg may import it.  It shares no code with the HIP
path; both sides receive the same inputs from ``synth``.

Every function here is pinned by CPU tests (closed forms, a hand-worked
example, invariants, finite differences and an independent library
cross-check); none is "parity unpinned".
"""
from .attention import *  # noqa: F401,F403
