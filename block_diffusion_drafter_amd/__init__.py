"""MI355X (gfx950) DFlash drafter: one parallel block-diffusion drafter pass.

The work runs in libdflash.so (hand-written HIP kernels behind the C ABI of
include/dflash.h); ``binding`` is its thin Python wrapper over torch device
memory and streams.
"""
from . import binding
from .binding import DraftModel, KVCache, accept, DFlashError

__all__ = ["binding", "DraftModel", "KVCache", "accept", "DFlashError"]
