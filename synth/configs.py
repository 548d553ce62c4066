"""Shapes of the drafter and of the workloads it is exercised on.

Pure data: sizes, dtypes and seeds. Nothing here computes any step of the
drafter pass. Both the HIP library's tests/bench and the CPU oracle read these
shapes; neither side's arithmetic lives here.

Shapes follow the workloads the DFlash pages describe: Qwen3-8B-shaped and
LLaMA-3.1-8B-shaped drafters with 5 draft layers, block 16 for Qwen3 targets,
5 target-layer features, concurrency 1-32 and contexts up to 32K tokens. The
MLP form, head counts, eps and RoPE theta are not printed on the pages; they
are the ones of the named target families.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class DrafterConfig:
    name: str
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    n_layers: int
    intermediate: int
    n_target_feats: int
    target_hidden: int
    vocab: int
    block_size: int
    rms_eps: float
    rope_theta: Optional[float]  # None: no rotary embedding (used by invariance checks)
    dtype: str                   # "fp32" or "bf16": storage/compute type of the GPU path
    tied_embeddings: bool        # embedding table and LM head are the same matrix
    sliding_window: int = 0      # > 0: attention window of the layers in sliding_layers
    sliding_layers: Tuple[int, ...] = ()

    @property
    def mask_token_id(self) -> int:
        # The MASK id is not printed on the pages; the synthetic drafters
        # reserve the last vocabulary entry for it.
        return self.vocab - 1

    @property
    def group(self) -> int:
        return self.n_heads // self.n_kv_heads

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def concat_width(self) -> int:
        return self.n_target_feats * self.target_hidden

    def with_(self, **kw) -> "DrafterConfig":
        return replace(self, **kw)


TINY_FP32 = DrafterConfig(
    name="tiny-fp32", hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, n_layers=1,
    intermediate=768, n_target_feats=3, target_hidden=256, vocab=1000, block_size=4,
    rms_eps=1e-6, rope_theta=1e4, dtype="fp32", tied_embeddings=True)

QWEN3_8B_SHAPED = DrafterConfig(
    name="qwen3-8b-shaped", hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128,
    n_layers=5, intermediate=12288, n_target_feats=5, target_hidden=4096, vocab=151936,
    block_size=16, rms_eps=1e-6, rope_theta=1e6, dtype="bf16", tied_embeddings=False)

LLAMA31_8B_SHAPED = DrafterConfig(
    name="llama3.1-8b-shaped", hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128,
    n_layers=5, intermediate=14336, n_target_feats=5, target_hidden=4096, vocab=128256,
    block_size=16, rms_eps=1e-6, rope_theta=5e5, dtype="bf16", tied_embeddings=False)

# Small bf16 drafter used only by the parity tests: it keeps the 8B-shaped head
# geometry (head_dim 128, 4 query heads per KV head, block 16) but shrinks every
# width so that the fp64 oracle finishes in well under a second, while the
# GEMMs still span several tiles and ragged tails (vocab 1000 is not a multiple
# of 16, 64 or 128).
SMALL_BF16 = DrafterConfig(
    name="small-bf16", hidden=512, n_heads=8, n_kv_heads=2, head_dim=128, n_layers=2,
    intermediate=1408, n_target_feats=3, target_hidden=384, vocab=1000, block_size=16,
    rms_eps=1e-6, rope_theta=1e6, dtype="bf16", tied_embeddings=False)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: a drafter plus batch, context and round structure."""
    name: str
    model: DrafterConfig
    batch: int
    ctx_len: Tuple[int, int]          # inclusive range; (n, n) for a fixed length
    rounds: int = 1
    append_new: Optional[Tuple[int, int]] = None   # rows appended before the forward
    plant_accept: bool = False        # targets planted so the true accept length is U{0..B-1}
    seeds: dict = field(default_factory=lambda: dict(
        weights=0, hiddens=1, ctx_lens=2, targets=3, round_base=1000))


WORKLOADS = {
    "tiny": Workload("tiny-fp32-b1-ctx32", TINY_FP32, batch=1, ctx_len=(32, 32)),
    "q1": Workload("qwen3-8b-shaped-b1-ctx2048", QWEN3_8B_SHAPED, batch=1, ctx_len=(2048, 2048)),
    "q32": Workload("qwen3-8b-shaped-b32-ctx512-8192", QWEN3_8B_SHAPED, batch=32,
                    ctx_len=(512, 8192), plant_accept=True),
    "q4l": Workload("qwen3-8b-shaped-b4-ctx32768-append", QWEN3_8B_SHAPED, batch=4,
                    ctx_len=(32768, 32768), append_new=(1, 16)),
    "l16": Workload("llama3.1-8b-shaped-b16-64rounds", LLAMA31_8B_SHAPED, batch=16,
                    ctx_len=(1024, 4096), rounds=64, plant_accept=True),
}
