"""fp64 CPU oracle of the Jamba Mamba-1 mixer.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It shares
no code with the HIP library and never imports it.
"""

from .mixer import *  # noqa: F401,F403
from .mixer import __all__  # noqa: F401
