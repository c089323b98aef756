"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This package only draws random numbers and packs them into arrays.  It holds
none of the method's arithmetic: no plane selection, no attention, no commit
rule and no byte layout.
"""
from .synth import *  # noqa: F401,F403
from .accept_inputs import *  # noqa: F401,F403
