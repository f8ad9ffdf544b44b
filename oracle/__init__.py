"""Float64 CPU oracle of the SP-TP linear layer.  Test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
package.  It shares no code with the HIP library.
"""
from .sptl_oracle import *  # noqa: F401,F403
