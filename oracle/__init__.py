"""CPU oracle (float64 NumPy) for Monarch-factored video attention.

Test infrastructure only: imported by the tests, the package smoke check and
the bench's CPU-baseline leg, never by the HIP library or its binding.
"""
from . import monarch_backward  # noqa: F401
from . import monarch_causal  # noqa: F401
from .monarch import *  # noqa: F401,F403
from .monarch import __all__ as _forward_all
from .monarch_backward import *  # noqa: F401,F403
from .monarch_backward import __all__ as _backward_all
from .monarch_causal import *  # noqa: F401,F403
from .monarch_causal import __all__ as _causal_all

__all__ = list(_forward_all) + list(_backward_all) + list(_causal_all)
