"""CPU oracle (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package.
The product path (token_filtered_backward_amd) never does, and this package imports nothing from it.
"""
from .collider_oracle import *  # noqa: F401,F403
