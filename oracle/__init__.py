"""CPU oracle for the GrowPage capacity-boundary event.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the library or its binding.
"""
from .reference import *  # noqa: F401,F403
from .reference import OracleConfig, GROW, COMPRESS, SHRINK  # noqa: F401
