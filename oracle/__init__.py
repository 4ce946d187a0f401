"""fp64 CPU oracle of the PR-Sink hot path.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its binding.
"""
from .prsink_oracle import *  # noqa: F401,F403
from .prsink_oracle import PRSinkOracle  # noqa: F401
