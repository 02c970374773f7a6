"""Test-infrastructure oracle (CPU, float64). Not part of the product path.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg import it.
"""
from .paged_attention import *  # noqa: F401,F403
