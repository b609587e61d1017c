"""CPU oracle for the sparse MoE layer forward (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this package.  The GPU library never imports, links or calls it, and the
oracle imports nothing from the GPU package.
"""
from .moe_oracle import *  # noqa: F401,F403
