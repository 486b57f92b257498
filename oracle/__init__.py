"""CPU oracle (test infrastructure only): plain float64 numpy definitions of the SSA
attention forward.  Imported by tests, the smoke check and the benchmark's CPU
baseline; never by the product path."""
from .ssa_oracle import *  # noqa: F401,F403
