"""CPU oracle for the DFlash drafter pass -- test infrastructure only.

Imported only by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg. The HIP library and its Python binding never import it; it imports
nothing from them.
"""
from . import dflash_oracle
from .dflash_oracle import *  # noqa: F401,F403
