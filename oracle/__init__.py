"""fp64 CPU oracle of the Jamba Mamba-1 mixer, of the whole Mamba layer around it, of their serving-style
calls (packed variable-length prefill, pooled states) and of the selective scan's backward pass.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It shares
no code with the HIP library and never imports it.
"""

from .backward import *  # noqa: F401,F403
from .backward import __all__ as _backward_all
from .layer import *  # noqa: F401,F403
from .layer import __all__ as _layer_all
from .mixer import *  # noqa: F401,F403
from .mixer import __all__ as _mixer_all
from .serving import *  # noqa: F401,F403
from .serving import __all__ as _serving_all

__all__ = list(_mixer_all) + list(_layer_all) + list(_serving_all) + list(_backward_all)
