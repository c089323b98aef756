"""Float64 CPU oracle for RIPE verify attention and commit.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the library.
"""
from .ripe_oracle import (DEEPEST, FULL, RIPE, LogicalCache, attend, commit, fill_prefix,  # noqa: F401
                          gather_prefix, layout_code, memory_positions, plane_select, verify)
from .layout import decode, encode, layout_bytes, layout_elements, ring_width  # noqa: F401
