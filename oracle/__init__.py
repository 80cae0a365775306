"""Float64 CPU oracle of the GCA hot path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library.
"""

from . import gca_oracle, condition, gumbel, offload, swa  # noqa: F401
from .gca_oracle import *  # noqa: F401,F403
