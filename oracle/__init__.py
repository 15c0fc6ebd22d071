"""The oracle: a plain, slow, fp64 CPU reference for the BaKron rounding pipeline.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import it. It shares no code with the HIP library.
"""
from .reference import *  # noqa: F401,F403
from .reference import __all__  # noqa: F401
