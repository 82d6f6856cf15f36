"""CPU oracle of the SureLock decoding step: test infrastructure, not product code.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  It shares no code with the HIP library.
"""
from .surelock_oracle import *  # noqa: F401,F403
