"""CPU oracle for the training-pattern attention of the drafter -- TEST
INFRASTRUCTURE, NOT PRODUCT CODE.

Only the tests, the package's smoke entry point and the benchmark's CPU leg
may import this module; the HIP library never imports, links or calls it, and
nothing here comes from the HIP side.

What is computed, with the passages it follows:

  [W] "DFlash: Block Diffusion for Flash Speculative Decoding" (wikillm
      summary), "Training" step 4 and the training-loss pseudocode: the blocks
      drawn from one sequence are packed into a single sequence and trained in
      one pass; a token attends, in both directions, to every position of its
      own block and to the injected context features, never to another block.
  [R] "DFlash: Why a Diffusion Drafter Can Accelerate an Autoregressive Model"
      (technical review), sec. 6.1: each sampled anchor becomes the clean first
      token of a block of B positions; the mask must hide the target features
      of positions after the anchor, and blocks must stay isolated.

Readings taken where the pages are silent (each repeated at its use):
  * T1 the block of anchor position a occupies sequence positions a .. a+B-1
    (rotary positions, as in decoding where the anchor sits right after the
    last context entry);
  * T2 the legal context of that block is the target features of positions
    0 .. a-1: the anchor's own feature is not used, exactly as at inference,
    where the context ends right before the anchor (ctx_len = a);
  * T3 scale 1/sqrt(head_dim), query head j reads KV head j // (Hq / Hkv), as
    in the decoding pass; the context K/V are the same per-layer projections
    of the fused features the decoding pass caches.

Parity status: pinned by tests/test_training_oracle.py against a dense masked
attention over the whole packed sequence computed by a library routine
(torch scaled_dot_product_attention with an explicit mask built from T1-T3),
against bidirectional attention for anchor 0, and against isolation
invariants; no printed worked example exists on the pages.
"""
from typing import Sequence

import numpy as np

from .dflash_oracle import kv_injected_attention

F64 = np.float64


def packed_block_attention(q, k_blk, v_blk, k_ctx, v_ctx, anchors: Sequence[int],
                           group: int) -> np.ndarray:
    """Attention of every packed block of one sequence ([W] "Training" step 4;
    [R] sec. 6.1).

    q      [nb, B, Hq, hd]  block queries (already normed and rotated)
    k_blk  [nb, B, Hkv, hd] block keys, v_blk likewise
    k_ctx  [Hkv, n, hd]     context keys of the sequence at positions 0..n-1
    v_ctx  [Hkv, n, hd]
    anchors[nb]             anchor position of each block, 0 <= a <= n

    Block j attends to its own B keys and to the context rows 0 .. a_j - 1
    (readings T1-T2): the decoding pass's attention with ctx_len = a_j.
    Returns [nb, B, Hq, hd] in float64.
    """
    nb, B, hq, hd = q.shape
    out = np.empty((nb, B, hq, hd), dtype=F64)
    for j in range(nb):
        a = int(anchors[j])
        if not 0 <= a <= k_ctx.shape[1]:
            raise ValueError(f"anchor {a} outside the context of {k_ctx.shape[1]} positions")
        out[j] = kv_injected_attention(q[j], k_blk[j], v_blk[j], k_ctx[:, :a], v_ctx[:, :a], group)
    return out
