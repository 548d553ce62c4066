"""Pins of the training-pattern attention oracle (oracle/training.py), none of
which re-runs its formula:

  * a dense masked attention over the whole packed sequence -- context rows
    then every block's rows as keys, the mask of readings T1-T2 built
    explicitly -- by torch's scaled_dot_product_attention (library routine);
  * anchor 0: bidirectional attention over the block alone (library routine);
  * isolation: another block's keys, context rows at or after the anchor, and
    nothing else may be changed without changing a block's output;
  * planted mistakes (the anchor's own feature visible, blocks seeing each
    other, a causal mask inside the block) that the dense pin must catch.
"""
import numpy as np
import pytest
import torch

from oracle import training as TR
from oracle import dflash_oracle as O


def inputs(seed, nb=5, B=4, hq=4, hkv=2, hd=16, n=40, anchors=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((nb, B, hq, hd))
    kb = rng.standard_normal((nb, B, hkv, hd))
    vb = rng.standard_normal((nb, B, hkv, hd))
    kc = rng.standard_normal((hkv, n, hd))
    vc = rng.standard_normal((hkv, n, hd))
    if anchors is None:
        anchors = np.sort(rng.integers(0, n + 1, size=nb))
    return q, kb, vb, kc, vc, np.asarray(anchors), hq // hkv


def dense_reference(q, kb, vb, kc, vc, anchors, group, ctx_inclusive=False, cross=False,
                    causal=False):
    """Packed sequence as one attention call: keys [context ; block 0 ; ... ;
    block nb-1], an explicit boolean mask per (query row, key)."""
    nb, B, hq, hd = q.shape
    n = kc.shape[1]
    L = nb * B
    Q = torch.tensor(q.reshape(L, hq, hd)).permute(1, 0, 2)                  # [hq, L, hd]
    Kall = np.concatenate([kc.transpose(1, 0, 2), kb.reshape(L, -1, hd)], 0)  # [n+L, hkv, hd]
    Vall = np.concatenate([vc.transpose(1, 0, 2), vb.reshape(L, -1, hd)], 0)
    K = torch.tensor(Kall).permute(1, 0, 2).repeat_interleave(group, 0)      # [hq, n+L, hd]
    V = torch.tensor(Vall).permute(1, 0, 2).repeat_interleave(group, 0)
    mask = np.zeros((L, n + L), dtype=bool)
    for j in range(nb):
        a = int(anchors[j])
        rows = slice(j * B, (j + 1) * B)
        mask[rows, :min(n, a + 1 if ctx_inclusive else a)] = True
        if cross:
            mask[rows, n:] = True
        else:
            mask[rows, n + j * B:n + (j + 1) * B] = True
        if causal:
            for i in range(B):
                mask[j * B + i, n + j * B + i + 1:n + (j + 1) * B] = False
    out = torch.nn.functional.scaled_dot_product_attention(
        Q, K, V, attn_mask=torch.tensor(mask), scale=1.0 / np.sqrt(hd))
    return out.permute(1, 0, 2).reshape(nb, B, hq, hd).numpy()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_packed_attention_equals_dense_masked_attention(seed):
    q, kb, vb, kc, vc, anc, g = inputs(seed)
    ours = TR.packed_block_attention(q, kb, vb, kc, vc, anc, g)
    ref = dense_reference(q, kb, vb, kc, vc, anc, g)
    np.testing.assert_allclose(ours, ref, atol=1e-11, rtol=1e-11)


def test_overlapping_and_edge_anchors():
    # anchors closer than B apart (overlapping spans), 0, and the full context
    q, kb, vb, kc, vc, anc, g = inputs(7, nb=4, anchors=[0, 2, 3, 40])
    ours = TR.packed_block_attention(q, kb, vb, kc, vc, anc, g)
    np.testing.assert_allclose(ours, dense_reference(q, kb, vb, kc, vc, anc, g), atol=1e-11)


def test_anchor_zero_is_bidirectional_attention_over_the_block():
    q, kb, vb, kc, vc, _, g = inputs(3, nb=1, anchors=[0])
    ours = TR.packed_block_attention(q, kb, vb, kc, vc, [0], g)[0]      # [B, hq, hd]
    Q = torch.tensor(q[0]).permute(1, 0, 2)
    K = torch.tensor(kb[0]).permute(1, 0, 2).repeat_interleave(g, 0)
    V = torch.tensor(vb[0]).permute(1, 0, 2).repeat_interleave(g, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(ours, ref, atol=1e-12)


def test_isolation():
    q, kb, vb, kc, vc, _, g = inputs(5, nb=3, anchors=[10, 20, 30])
    base = TR.packed_block_attention(q, kb, vb, kc, vc, [10, 20, 30], g)
    # another block's keys and values
    kb2, vb2 = kb.copy(), vb.copy()
    kb2[2] += 5.0
    vb2[2] -= 3.0
    out = TR.packed_block_attention(q, kb2, vb2, kc, vc, [10, 20, 30], g)
    np.testing.assert_array_equal(out[:2], base[:2])
    assert not np.allclose(out[2], base[2])
    # context rows at or after block 0's anchor, but before block 1's
    kc2 = kc.copy()
    kc2[:, 10:20] += 4.0
    out = TR.packed_block_attention(q, kb, vb, kc2, vc, [10, 20, 30], g)
    np.testing.assert_array_equal(out[0], base[0])
    assert not np.allclose(out[1], base[1]) and not np.allclose(out[2], base[2])
    # the last legal context row of block 0
    vc2 = vc.copy()
    vc2[:, 9] += 1.0
    out = TR.packed_block_attention(q, kb, vb, kc, vc2, [10, 20, 30], g)
    assert not np.allclose(out[0], base[0])


def test_one_block_equals_the_decoding_attention_at_that_context_length():
    # the training mask of a block is the decoding pass's with ctx_len = anchor
    q, kb, vb, kc, vc, _, g = inputs(9, nb=1, anchors=[17])
    ours = TR.packed_block_attention(q, kb, vb, kc, vc, [17], g)[0]
    ref = dense_reference(q[:1], kb[:1], vb[:1], kc[:, :17], vc[:, :17], [17], g)[0]
    np.testing.assert_allclose(ours, ref, atol=1e-11)
    with pytest.raises(ValueError):
        TR.packed_block_attention(q, kb, vb, kc, vc, [41], g)


@pytest.mark.parametrize("mistake", ["ctx_inclusive", "cross", "causal"])
def test_dense_pin_catches_planted_mistakes(mistake):
    q, kb, vb, kc, vc, anc, g = inputs(11, anchors=[3, 9, 15, 22, 30])
    ours = TR.packed_block_attention(q, kb, vb, kc, vc, anc, g)
    wrong = dense_reference(q, kb, vb, kc, vc, anc, g, **{mistake: True})
    assert np.abs(ours - wrong).max() > 1e-3
