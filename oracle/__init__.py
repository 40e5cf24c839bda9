"""fp64 CPU oracle for the MC-Sparse hot path (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  It shares no code with the HIP library and imports nothing from it.
"""
from .mcs_oracle import *  # noqa: F401,F403
from .mcs_oracle import default_scale  # noqa: F401
