"""fp64 CPU oracle of the LLoPS hot path -- TEST INFRASTRUCTURE.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
it. It shares no code with the HIP library and imports nothing from it.
"""
from .llops_oracle import *  # noqa: F401,F403
