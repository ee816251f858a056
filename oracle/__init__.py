"""CPU oracle (float64 NumPy) for Monarch-factored video attention.

Test infrastructure only: imported by the tests, the package smoke check and
the bench's CPU-baseline leg, never by the HIP library or its binding.
"""
from .monarch import *  # noqa: F401,F403
from .monarch import __all__  # noqa: F401
