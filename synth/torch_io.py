"""Move seeded host draws onto the GPU as torch tensors (storage conversion only)."""
from __future__ import annotations

from typing import Dict, List

import numpy as np
import torch

from .inputs import HostTensor, Weights


def to_device(t: HostTensor, device="cuda") -> torch.Tensor:
    if t.bf16:
        return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).view(
            torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(t.data)).to(device)


def weights_to_device(w: Weights, device="cuda", names: List[str] = None) -> Dict[str, torch.Tensor]:
    out = {}
    for n in (names or w.names()):
        out[n] = to_device(w.get(n), device)
    if w.cfg.tied_embeddings:
        out["lm_head"] = out["embed"]
    return out
