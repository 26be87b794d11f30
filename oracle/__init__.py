"""CPU oracle of the DiT hot path -- test infrastructure only.

Only tests/, the package smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the GPU library.
"""

from .dit_oracle import *  # noqa: F401,F403
