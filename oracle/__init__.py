"""fp64 CPU oracle of the DLite draft step (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  The product library never does.
"""
from .dlite_oracle import *  # noqa: F401,F403
