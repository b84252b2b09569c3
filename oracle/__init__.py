"""Float64 CPU oracle for speculative verification and the SAGUARO cache build.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package. The GPU library and its
Python binding never import it, and it shares no code with them.
"""
from .ssd_oracle import *  # noqa: F401,F403
from .ssd_oracle import __all__  # noqa: F401
