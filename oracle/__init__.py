"""CPU oracle (test infrastructure): only tests, the smoke check and the benchmark's CPU-baseline leg use it."""
from .rotattn_oracle import *  # noqa: F401,F403
from . import rotattn_oracle as core  # noqa: F401
