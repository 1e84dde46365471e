"""CPU oracle of the ForwardPass attention step (fp64, numpy).

Test infrastructure: imported only by tests/, the smoke check and the
benchmark's CPU-baseline leg; the HIP path never uses it.
"""

from .fp_oracle import *  # noqa: F401,F403
from . import fp_oracle  # noqa: F401
