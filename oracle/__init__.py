"""CPU oracle of the ShadowKV decode step (test infrastructure only).

Imported only by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg.
"""
from . import shadowkv  # noqa: F401
