"""CPU oracle for the stream-aware W4A8/W4A4 linear (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package.  The product path (the HIP library and its binding) never imports,
links or runs anything from here.  See rudder_oracle.c for the method, its
citations and the readings taken where the pages are silent.
"""
from .oracle import *  # noqa: F401,F403
from .oracle import __all__  # noqa: F401
from . import calibration  # noqa: F401
