"""CPU oracle for the routed-MoE expert layer (test infrastructure only).

Only tests/, ``__graft_entry__.smoke()`` and the CPU-baseline leg of bench.py
may import this package; the HIP library never does.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import local_expert  # noqa: F401
