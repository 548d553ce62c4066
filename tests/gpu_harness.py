"""Shared machinery of the GPU parity tests: run the HIP library through its
C ABI and the CPU oracle on the same seeded inputs, and compare.

Tolerances (written here once, used by every parity test):
  * fp32 drafter: max-abs error 1e-4 on context features, cached K/V, hidden
    states after every layer and logits;
  * bf16 drafter: normwise relative error max|gpu-ref| / max|ref| <= 3e-2 on
    the same tensors (the GPU rounds GEMM inputs, q/k/v, P and the cache to
    bf16; the oracle rounds nothing);
    The bound holds over the whole tensor and, separately, over every group
    along its leading axes (each sequence of a batch, each KV head of a cache
    slice), so an error confined to one short sequence or one head cannot hide
    under another's larger values;
  * draft token ids: bit-exact wherever the oracle's top-1/top-2 margin
    exceeds 0.05. At the other slots (near-ties) several tokens are correct
    drafts, and the GPU's pick must be one of them: the argmax of the GPU's own
    logits, whose oracle logit lies within max(0.05, 2 eps) of the oracle's
    top-1, eps being the row's measured max |gpu - oracle| logit error (a
    token beats the top-1 on the GPU only if the two differ by at most the sum
    of their errors); without GPU logits the bound is 0.05;
  * accept lengths and bonus tokens: the GPU's equal the prefix rule applied
    to its own drafts (every sequence), and equal the oracle's wherever the
    GPU's drafts agree with the oracle's on every position the prefix test
    reads (i <= min(a, B-2)); where they do not, the first differing position
    is a validated near-tie.
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


def group_rel_errors(got, ref, group_axes: int) -> np.ndarray:
    """Normwise error max|gpu-ref| / max|ref| of every group formed by the
    first group_axes axes (e.g. 1: per sequence of [b, ...])."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    lead = got.shape[:group_axes]
    g = got.reshape(int(np.prod(lead)), -1)
    r = ref.reshape(int(np.prod(lead)), -1)
    if g.shape[1] == 0:
        return np.zeros(g.shape[0])
    err = np.max(np.abs(g - r), axis=1)
    scale = np.max(np.abs(r), axis=1)
    return np.where(scale > 0, err / np.maximum(scale, 1e-30), np.where(err > 0, np.inf, 0.0))


def _check_close(cfg, got, ref, what: str, group_axes: int):
    a, r = err_stats(got, ref)
    worst = r
    if cfg.dtype == "fp32":
        assert a <= TOL_FP32_ABS, f"{what}: max-abs {a:.3e} > {TOL_FP32_ABS}"
    else:
        assert r <= TOL_BF16_REL, f"{what}: normwise rel {r:.3e} > {TOL_BF16_REL}"
        if group_axes > 0 and np.asarray(ref).size:
            per = group_rel_errors(got, ref, group_axes)
            worst = float(per.max())
            bad = np.argwhere(per.reshape(np.asarray(ref).shape[:group_axes]) > TOL_BF16_REL)
            assert not len(bad), (f"{what}: normwise rel {worst:.3e} > {TOL_BF16_REL} in group(s) "
                                  f"{bad[:5].tolist()}")
    return a, r, worst


def assert_close(cfg, got, ref, what: str, group_axes: int = 0) -> None:
    """fp32: max-abs bound. bf16: normwise bound over the tensor and over every
    group along the first group_axes axes."""
    a, r, worst = _check_close(cfg, got, ref, what, group_axes)
    log(f"  {what}: max-abs {a:.3e} rel {r:.3e}" +
        (f" (worst group {worst:.3e})" if group_axes > 0 and cfg.dtype != "fp32" else ""))


def assert_close_each(cfg, items, what: str, group_axes: int = 0) -> None:
    """assert_close on every (label, got, ref) of items (e.g. one per sequence,
    grouped per KV head); one log line with the worst figures."""
    wa = wr = ww = 0.0
    for label, got, ref in items:
        a, r, w = _check_close(cfg, got, ref, f"{what} {label}", group_axes)
        wa, wr, ww = max(wa, a), max(wr, r), max(ww, w)
    log(f"  {what}: {len(items)} parts, worst max-abs {wa:.3e} rel {wr:.3e}" +
        (f" (worst group {ww:.3e})" if group_axes > 0 and cfg.dtype != "fp32" else ""))


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


def check_drafts(res: O.ForwardResult, drafts_gpu: np.ndarray, what: str,
                 logits_gpu=None) -> int:
    """Every slot: bit-exact where the oracle's top-1/top-2 margin exceeds
    MARGIN; elsewhere the GPU's token must be a valid near-tie pick (see the
    module docstring). logits_gpu: the GPU's logits of the same rows
    ([b, B-1, V], tensor or array) when the call produced them. Returns the
    number of near-tie slots."""
    drafts_gpu = np.asarray(drafts_gpu, dtype=np.int64)
    V = res.logits.shape[-1]
    assert ((drafts_gpu >= 0) & (drafts_gpu < V)).all(), f"{what}: token ids out of range"
    ok = res.margins > MARGIN
    mism = (drafts_gpu != res.drafts) & ok
    assert not mism.any(), f"{what}: {int(mism.sum())} confident drafts differ at {np.argwhere(mism)[:5]}"
    top1 = np.take_along_axis(res.logits, res.drafts[..., None], -1)[..., 0]
    mine = np.take_along_axis(res.logits, drafts_gpu[..., None], -1)[..., 0]
    gap = top1 - mine
    bound = np.full(gap.shape, MARGIN)
    widened = 0
    if logits_gpu is not None:
        lg = logits_gpu.detach().float().cpu().numpy().astype(np.float64) \
            if isinstance(logits_gpu, torch.Tensor) else np.asarray(logits_gpu, dtype=np.float64)
        assert lg.shape == res.logits.shape, (lg.shape, res.logits.shape)
        # the GPU's token is the argmax of its own logits (lowest id on ties)
        own = np.argmax(lg, axis=-1)
        assert (own == drafts_gpu).all(), f"{what}: drafts are not the argmax of the GPU's logits"
        eps = np.max(np.abs(lg - res.logits), axis=-1)
        bound = np.maximum(MARGIN, 2.0 * eps)
        widened = int(((gap > MARGIN) & (gap <= bound)).sum())
    invalid = gap > bound
    assert not invalid.any(), (f"{what}: {int(invalid.sum())} near-tie slots hold a token whose "
                               f"oracle logit is further below the top-1 than the bound: "
                               f"{np.argwhere(invalid)[:5].tolist()}, gaps {gap[invalid][:5]}, "
                               f"bounds {bound[invalid][:5]}")
    excl = int((~ok).sum())
    differ = int(((drafts_gpu != res.drafts) & ~ok).sum())
    log(f"  {what}: drafts bit-exact on {int(ok.sum())}/{ok.size} confident slots; "
        f"{excl} near-tie slots (margin <= {MARGIN}) all hold a valid pick "
        f"({differ} differ from the oracle's argmax, {widened} of them beyond {MARGIN} but "
        f"within twice the row's logit error; 0 invalid)")
    return excl


def check_accept(res: O.ForwardResult, targets: np.ndarray, acc_gpu: np.ndarray,
                 bonus_gpu: np.ndarray, drafts_gpu: np.ndarray, what: str) -> int:
    """Accept lengths and bonus tokens: the prefix rule on the GPU's own drafts
    for every sequence; equal to the oracle's wherever the GPU's drafts agree
    with the oracle's on every position the prefix test reads. Where they do
    not, the first differing read position must be a near-tie (check_drafts
    has validated the GPU's token there). Returns the number of sequences
    compared with the oracle."""
    acc_o, bonus_o = O.accept(res.drafts, targets)
    b, m = res.drafts.shape
    checked = explained = 0
    for s in range(b):
        a = int(acc_o[s])
        a_own, b_own = O.accept(drafts_gpu[s:s + 1], targets[s:s + 1])
        assert acc_gpu[s] == a_own[0] and bonus_gpu[s] == b_own[0], f"{what}: seq {s} prefix rule"
        read = min(a, m - 1) + 1 if m else 0
        same = np.asarray(drafts_gpu[s, :read]) == res.drafts[s, :read]
        if same.all():
            assert acc_gpu[s] == a and bonus_gpu[s] == bonus_o[s], (
                f"{what}: seq {s} accept {acc_gpu[s]} bonus {bonus_gpu[s]} vs oracle {a} "
                f"{bonus_o[s]}")
            checked += 1
        else:
            i = int(np.argmin(same))
            assert res.margins[s, i] <= MARGIN, f"{what}: seq {s} differs at confident slot {i}"
            explained += 1
    log(f"  {what}: accept lengths equal to the oracle's on {checked}/{b} sequences; "
        f"{explained} differ through a near-tie draft read by the prefix test")
    return checked
