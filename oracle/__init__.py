"""CPU oracle (test infrastructure only; never on the product path).

Only the test suite, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  See loco_oracle for the definitions and their sources.
"""
from .loco_oracle import *  # noqa: F401,F403
from .loco_oracle import __all__  # noqa: F401
