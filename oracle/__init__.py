"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .ref import *  # noqa: F401,F403
from .ref import GROUP, REL_TOL, ABS_TOL  # noqa: F401
