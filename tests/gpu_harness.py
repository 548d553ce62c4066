"""Shared machinery of the GPU parity tests: run the HIP library through its
C ABI and the CPU oracle on the same seeded inputs, and compare.

Tolerances (written here once, used by every parity test):
  * fp32 drafter: max-abs error 1e-4 on context features, cached K/V, hidden
    states after every layer and logits;
  * bf16 drafter: normwise relative error max|gpu-ref| / max|ref| <= 3e-2 on
    the same tensors (the GPU rounds GEMM inputs, q/k/v, P and the cache to
    bf16; the oracle rounds nothing);
  * draft token ids bit-exact wherever the oracle's top-1 minus top-2 logit
    margin exceeds 0.05; accept lengths bit-exact wherever every position the
    prefix test reads (i <= min(a, B-2)) has such a margin. Excluded positions
    are counted and must stay a minority.
"""
from __future__ import annotations

import sys
import time
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

from block_diffusion_drafter_amd import binding as B
from oracle import dflash_oracle as O
from synth import inputs as I
from synth import torch_io

MARGIN = 0.05
TOL_FP32_ABS = 1e-4
TOL_BF16_REL = 3e-2


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def err_stats(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0, 0.0
    abs_err = float(np.max(np.abs(got - ref)))
    scale = float(np.max(np.abs(ref)))
    return abs_err, abs_err / max(scale, 1e-30)


def assert_close(cfg, got, ref, what: str) -> None:
    a, r = err_stats(got, ref)
    if cfg.dtype == "fp32":
        assert a <= TOL_FP32_ABS, f"{what}: max-abs {a:.3e} > {TOL_FP32_ABS}"
    else:
        assert r <= TOL_BF16_REL, f"{what}: normwise rel {r:.3e} > {TOL_BF16_REL}"
    log(f"  {what}: max-abs {a:.3e} rel {r:.3e}")


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def prefix_offsets(counts) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def capacity_for(max_ctx: int, block: int, extra: int = 0) -> int:
    need = max_ctx + block + extra
    return ((need + 31) // 32) * 32


@dataclass
class Model:
    cfg: object
    host: I.Weights
    gpu: B.DraftModel
    oracle_w: dict


_MODELS = {}


def build_model(cfg, seed: int = 0) -> Model:
    """Seeded drafter on both sides; the last full-size one is reused across tests."""
    key = (cfg, seed)
    if key in _MODELS:
        return _MODELS[key]
    if cfg.hidden >= 2048:
        _MODELS.clear()
        log(f"  drawing {cfg.name} weights")
    host = I.Weights(cfg, seed)
    dev = torch_io.weights_to_device(host)
    gpu = B.DraftModel(cfg, dev)
    # fp32 views of the exact stored values; the oracle widens them to fp64.
    ow = {n: host.get(n).f32() for n in host.names()}
    if cfg.tied_embeddings:
        ow["lm_head"] = ow["embed"]
    model = Model(cfg, host, gpu, ow)
    if cfg.hidden >= 2048:
        _MODELS[key] = model
    return model


def feats_to_device(feats: List[I.HostTensor]) -> List[torch.Tensor]:
    return [torch_io.to_device(f) for f in feats]


def check_drafts(res: O.ForwardResult, drafts_gpu: np.ndarray, what: str) -> int:
    ok = res.margins > MARGIN
    mism = (drafts_gpu != res.drafts) & ok
    assert not mism.any(), f"{what}: {int(mism.sum())} confident drafts differ at {np.argwhere(mism)[:5]}"
    excl = int((~ok).sum())
    log(f"  {what}: drafts bit-exact on {int(ok.sum())}/{ok.size} confident slots "
        f"({excl} excluded, margin <= {MARGIN})")
    return excl


def check_accept(res: O.ForwardResult, targets: np.ndarray, acc_gpu: np.ndarray,
                 bonus_gpu: np.ndarray, drafts_gpu: np.ndarray, what: str) -> int:
    acc_o, bonus_o = O.accept(res.drafts, targets)
    m = res.drafts.shape[1]
    checked = 0
    for s in range(len(acc_o)):
        a = int(acc_o[s])
        # Property at any margin: the GPU's accept length is the longest
        # matching prefix of its own drafts against the targets.
        a_own, b_own = O.accept(drafts_gpu[s:s + 1], targets[s:s + 1])
        assert acc_gpu[s] == a_own[0] and bonus_gpu[s] == b_own[0], f"{what}: seq {s} prefix rule"
        if (res.margins[s, :min(a, m - 1) + 1] > MARGIN).all() or m == 0:
            assert acc_gpu[s] == a and bonus_gpu[s] == bonus_o[s], (
                f"{what}: seq {s} accept {acc_gpu[s]} vs oracle {a}")
            checked += 1
    log(f"  {what}: accept lengths bit-exact on {checked}/{len(acc_o)} confident sequences")
    return checked
