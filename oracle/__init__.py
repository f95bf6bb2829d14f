"""Test infrastructure: the plain fp64 CPU oracle for OAL causal attention.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
this package.  The product path (the HIP library and its Python binding) never
imports or calls it, and it shares no code with that path.
"""

from .oal_oracle import *  # noqa: F401,F403
