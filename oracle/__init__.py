"""CPU float64 oracle for the HARP rotated low-bit linear.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the library in rotated_bit_amd/.
"""
from . import harp_oracle  # noqa: F401
from .harp_oracle import *  # noqa: F401,F403
