"""Seeded synthetic inputs for the drafter pass.

This module only draws numbers: random-init drafter weights, target hidden
states, context lengths, cached context keys/values and target block tokens.
It performs no step of the drafter pass; both the HIP path's tests and the CPU
oracle consume what it produces.

Recipe (all seeds fixed, see ``Workload.seeds``):
  * weight matrices ~ N(0, 0.02^2) (0.02 is the standard deviation); RMSNorm
    gains are 1.0. Each tensor has its own stream derived from
    (weights seed, tensor name), so one tensor can be drawn without the others.
  * target hidden states ~ N(0, 1).
  * values are drawn in fp32; for bf16 drafters they are rounded to bf16 with
    round-to-nearest-even and both sides consume exactly those bits.
  * token ids are uniform on [0, vocab-1), so the MASK id (vocab-1) never
    appears as a drawn token.
  * cached context keys ~ N(0, 1) and values ~ N(0, (0.02*sqrt(hidden))^2):
    the scale that per-head RMSNorm (gain 1) gives keys, and that a N(0, 0.02^2)
    value projection gives an RMS-normalised context feature.

Large tensors are drawn in fixed 4M-element chunks, each from its own child
seed, on a thread pool; the result does not depend on the number of threads.
"""
from __future__ import annotations

import os
import zlib
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence

import numpy as np

from .configs import DrafterConfig, Workload

_CHUNK = 1 << 22
WEIGHT_STD = 0.02


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _seed_seq(seed: int, name: str) -> np.random.SeedSequence:
    return np.random.SeedSequence([int(seed), zlib.crc32(name.encode())])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even); returns uint16 bits.
    Inputs here are finite draws, so no NaN handling is needed."""
    # For finite fp32 the largest pattern is 0xFF7FFFFF, so adding at most
    # 0x8000 cannot wrap a uint32.
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(seed: int, name: str, shape: Sequence[int], std: float, bf16: bool) -> np.ndarray:
    """N(0, std^2) draws of ``shape``; uint16 bf16 bits if ``bf16`` else fp32."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)
    children = _seed_seq(seed, name).spawn(nchunks)

    def work(i: int) -> None:
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(children[i]))
        v = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[lo:hi] = f32_to_bf16_bits(v) if bf16 else v

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(tuple(shape))


class HostTensor:
    """A host array in its storage form (fp32 values or bf16 bits)."""

    def __init__(self, data: np.ndarray, bf16: bool):
        self.data = data
        self.bf16 = bf16

    @property
    def shape(self):
        return self.data.shape

    def f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.data) if self.bf16 else self.data

    def f64(self) -> np.ndarray:
        return self.f32().astype(np.float64)


def layer_tensor_names(l: int) -> List[str]:
    return [f"layers.{l}.{n}" for n in
            ("in_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "post_norm",
             "w_gate", "w_up", "w_down")]


def weight_shapes(cfg: DrafterConfig) -> Dict[str, tuple]:
    d, hd = cfg.hidden, cfg.head_dim
    s = {"embed": (cfg.vocab, d), "fc": (d, cfg.concat_width), "fc_norm": (d,),
         "final_norm": (d,)}
    if not cfg.tied_embeddings:
        s["lm_head"] = (cfg.vocab, d)
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        s[p + "in_norm"] = (d,)
        s[p + "wq"] = (cfg.q_dim, d)
        s[p + "wk"] = (cfg.kv_dim, d)
        s[p + "wv"] = (cfg.kv_dim, d)
        s[p + "q_norm"] = (hd,)
        s[p + "k_norm"] = (hd,)
        s[p + "wo"] = (d, cfg.q_dim)
        s[p + "post_norm"] = (d,)
        s[p + "w_gate"] = (cfg.intermediate, d)
        s[p + "w_up"] = (cfg.intermediate, d)
        s[p + "w_down"] = (d, cfg.intermediate)
    return s


def _is_gain(name: str) -> bool:
    return name.endswith("norm")


class Weights:
    """Seeded random-init drafter weights, drawn lazily per tensor."""

    def __init__(self, cfg: DrafterConfig, seed: int = 0):
        self.cfg = cfg
        self.seed = seed
        self.shapes = weight_shapes(cfg)
        self._cache: Dict[str, HostTensor] = {}

    def names(self) -> List[str]:
        return list(self.shapes)

    def get(self, name: str) -> HostTensor:
        if name == "lm_head" and self.cfg.tied_embeddings:
            return self.get("embed")
        t = self._cache.get(name)
        if t is None:
            bf16 = self.cfg.dtype == "bf16"
            shape = self.shapes[name]
            if _is_gain(name):
                one = np.ones(shape, np.float32)
                t = HostTensor(f32_to_bf16_bits(one) if bf16 else one, bf16)
            else:
                t = HostTensor(normal(self.seed, name, shape, WEIGHT_STD, bf16), bf16)
            self._cache[name] = t
        return t

    def __getitem__(self, name: str) -> HostTensor:
        return self.get(name)

    def set(self, name: str, values_f32: np.ndarray) -> None:
        """Replace a tensor (used by invariance checks that build related models)."""
        bf16 = self.cfg.dtype == "bf16"
        v = np.ascontiguousarray(values_f32, dtype=np.float32)
        self._cache[name] = HostTensor(f32_to_bf16_bits(v) if bf16 else v, bf16)

    def f64_dict(self) -> Dict[str, np.ndarray]:
        """Every tensor widened to fp64 (tiny and small drafters only)."""
        out = {n: self.get(n).f64() for n in self.names()}
        if self.cfg.tied_embeddings:
            out["lm_head"] = out["embed"]
        return out

    def drop(self, name: Optional[str] = None) -> None:
        if name is None:
            self._cache.clear()
        else:
            self._cache.pop(name, None)


def target_hiddens(cfg: DrafterConfig, n_rows: int, seed: int, tag: str = "prefill"
                   ) -> List[HostTensor]:
    """n_target_feats arrays [n_rows, target_hidden] of N(0,1) target features."""
    bf16 = cfg.dtype == "bf16"
    return [HostTensor(normal(seed, f"hidden.{tag}.{f}", (n_rows, cfg.target_hidden), 1.0, bf16),
                       bf16) for f in range(cfg.n_target_feats)]


def ctx_lengths(w: Workload) -> np.ndarray:
    lo, hi = w.ctx_len
    if lo == hi:
        return np.full(w.batch, lo, dtype=np.int32)
    g = np.random.Generator(np.random.PCG64(_seed_seq(w.seeds["ctx_lens"], "ctx_lens")))
    return g.integers(lo, hi + 1, size=w.batch).astype(np.int32)


def append_counts(w: Workload, seed_tag: str = "append") -> np.ndarray:
    lo, hi = w.append_new
    g = np.random.Generator(np.random.PCG64(_seed_seq(w.seeds["ctx_lens"], seed_tag)))
    return g.integers(lo, hi + 1, size=w.batch).astype(np.int32)


def uniform_tokens(cfg: DrafterConfig, shape, seed: int, tag: str) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(_seed_seq(seed, tag)))
    return g.integers(0, cfg.vocab - 1, size=shape).astype(np.int32)


def planted_accept_lengths(n: int, m: int, seed: int, tag: str) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(_seed_seq(seed, "plant." + tag)))
    return g.integers(0, m + 1, size=n).astype(np.int32)


def plant_targets(drafts: np.ndarray, a_star: np.ndarray, vocab: int, seed: int, tag: str
                  ) -> np.ndarray:
    """Target block tokens [b, B] whose longest agreement with ``drafts`` [b, B-1]
    is exactly ``a_star`` [b]: t[:a] = d[:a], t[a] != d[a] (if a < B-1), the rest
    uniform. Input construction only; the drafts come from the oracle."""
    b, m = drafts.shape
    g = np.random.Generator(np.random.PCG64(_seed_seq(seed, "targets." + tag)))
    t = g.integers(0, vocab - 1, size=(b, m + 1)).astype(np.int32)
    for s in range(b):
        a = int(a_star[s])
        t[s, :a] = drafts[s, :a]
        if a < m and t[s, a] == drafts[s, a]:
            t[s, a] = (drafts[s, a] + 1) % (vocab - 1)
    return t


def anchors(cfg: DrafterConfig, batch: int, seed: int, tag: str = "anchor") -> np.ndarray:
    return uniform_tokens(cfg, (batch,), seed, tag)


def cache_state(cfg: DrafterConfig, ctx_lens: Sequence[int], seed: int
                ) -> List[List[tuple]]:
    """Synthetic cached context K/V: [layer][seq] -> (K, V) HostTensors of shape
    [n_kv_heads, ctx_len, head_dim]. Keys N(0,1); values N(0, (0.02*sqrt(d))^2)."""
    bf16 = cfg.dtype == "bf16"
    v_std = WEIGHT_STD * float(np.sqrt(cfg.hidden))
    out = []
    for l in range(cfg.n_layers):
        row = []
        for s, c in enumerate(ctx_lens):
            shp = (cfg.n_kv_heads, int(c), cfg.head_dim)
            k = HostTensor(normal(seed, f"cache.k.{l}.{s}", shp, 1.0, bf16), bf16)
            v = HostTensor(normal(seed, f"cache.v.{l}.{s}", shp, v_std, bf16), bf16)
            row.append((k, v))
        out.append(row)
    return out


def training_anchors(ctx_len: int, n_blocks: int, prompt_len: int, seed: int, tag: str
                     ) -> np.ndarray:
    """Sorted anchor positions of one training sequence, uniform over its
    response part [prompt_len, ctx_len] (drawn with replacement, so blocks may
    start closer than B apart, as independent draws do)."""
    g = np.random.Generator(np.random.PCG64(_seed_seq(seed, "train.anchors." + tag)))
    return np.sort(g.integers(prompt_len, ctx_len + 1, size=n_blocks)).astype(np.int32)


def packed_block_qkv(cfg: DrafterConfig, n_blk: int, seed: int, tag: str) -> List[HostTensor]:
    """Synthetic packed-block queries [n_blk, B, Hq, hd] and keys / values
    [n_blk, B, Hkv, hd], N(0,1) (the scale of RMS-normed heads)."""
    bf16 = cfg.dtype == "bf16"
    B, hd = cfg.block_size, cfg.head_dim
    shp = {"q": (n_blk, B, cfg.n_heads, hd), "k": (n_blk, B, cfg.n_kv_heads, hd),
           "v": (n_blk, B, cfg.n_kv_heads, hd)}
    return [HostTensor(normal(seed, f"train.{n}.{tag}", shp[n], 1.0, bf16), bf16)
            for n in ("q", "k", "v")]
