"""Training-pattern attention of packed blocks through the C ABI
(dflash_packed_block_attention) against the oracle (oracle/training.py):
context K/V written by the library's own fusion + injection path from seeded
features (and by the oracle's from the same features), seeded block
queries/keys/values, anchors drawn over each sequence's response. Edge cases:
anchor 0 (the block alone), anchor at the end of the context, blocks closer
than B apart, anchors past the context (clamped and flagged). The
Qwen3-8B-shaped case compares sampled blocks (the oracle runs one block at a
time)."""
import numpy as np
import pytest
import torch

from gpu_harness import (assert_close, build_model, capacity_for, feats_to_device, log,
                         prefix_offsets, to_np)
from oracle import dflash_oracle as O
from oracle import training as TR
from synth import QWEN3_8B_SHAPED, SMALL_BF16, TINY_FP32
from synth import inputs as I
from synth import torch_io

pytestmark = pytest.mark.gpu


def prefill(M, cfg, ctx_lens, tag):
    """Context of every sequence through ctx_project + ctx_kv_append; the
    oracle's caches from the same features."""
    b, d = len(ctx_lens), cfg.hidden
    n_tot = int(sum(ctx_lens))
    cap = capacity_for(max(ctx_lens), cfg.block_size)
    feats = I.target_hiddens(cfg, n_tot, seed=1, tag=tag)
    ws = M.gpu.new_workspace(b, cap, n_tot)
    ctx = torch.empty((n_tot, d), dtype=M.gpu.dtype, device="cuda")
    cache = M.gpu.new_cache(b, cap)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    M.gpu.ctx_project(feats_to_device(feats), ctx, ws)
    M.gpu.ctx_kv_append(cache, ctx, torch.from_numpy(prefix_offsets(ctx_lens)).cuda(), ws, status)
    torch.cuda.synchronize()
    assert status.item() == 0
    ow = M.oracle_w
    ctx_o = O.ctx_project([f.f32() for f in feats], ow["fc"], ow["fc_norm"], cfg.rms_eps)
    cu = prefix_offsets(ctx_lens)
    caches = [O.prefill_cache(ctx_o[cu[s]:cu[s + 1]], 0, ow, cfg) for s in range(b)]
    return cache, caches


def run_packed(cfg, ctx_lens, anchors, tag, layers=None, sample=None, expect_flag=False):
    ctx_lens = [int(c) for c in ctx_lens]
    anchors = np.asarray(anchors, dtype=np.int32)
    n_seq, nb = anchors.shape
    log(f"case: {cfg.name} packed attention, {n_seq} x {nb} blocks, ctx {ctx_lens} ({tag})")
    M = build_model(cfg)
    cache, caches = prefill(M, cfg, ctx_lens, tag)
    qh, kh, vh = I.packed_block_qkv(cfg, n_seq * nb, seed=5, tag=tag)
    q, kb, vb = (torch_io.to_device(t) for t in (qh, kh, vh))
    B = cfg.block_size
    shp_q = (n_seq, nb, B, cfg.n_heads, cfg.head_dim)
    shp_kv = (n_seq, nb, B, cfg.n_kv_heads, cfg.head_dim)
    q, kb, vb = q.view(shp_q), kb.view(shp_kv), vb.view(shp_kv)
    out = torch.full(shp_q, float("nan"), dtype=q.dtype, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    anc_g = torch.from_numpy(anchors).cuda()
    qo, ko, vo = (t.f32().reshape(s) for t, s in ((qh, shp_q), (kh, shp_kv), (vh, shp_kv)))
    group = cfg.n_heads // cfg.n_kv_heads
    for l in (layers if layers is not None else range(cfg.n_layers)):
        M.gpu.packed_block_attention(cache, l, anc_g, q, kb, vb, out, status)
        torch.cuda.synchronize()
        assert (status.item() != 0) == expect_flag, f"device status {status.item()}"
        got = to_np(out)
        for s in range(n_seq):
            blocks = range(nb) if sample is None else sample
            a = np.minimum(anchors[s], ctx_lens[s])
            ref = TR.packed_block_attention(qo[s][list(blocks)], ko[s][list(blocks)],
                                            vo[s][list(blocks)], caches[s].k[l], caches[s].v[l],
                                            a[list(blocks)], group)
            assert_close(cfg, got[s][list(blocks)], ref, f"layer {l} seq {s} packed attention")


def test_gpu_packed_tiny_fp32():
    # block 4: overlapping anchors, anchor 0 and the full context
    run_packed(TINY_FP32, [32, 40], [[0, 1, 3, 17, 32], [2, 2, 20, 39, 40]], "tiny")


def test_gpu_packed_small_bf16_ragged():
    cfg = SMALL_BF16
    ctx = [300, 77]
    anc = np.stack([I.training_anchors(c, 24, c // 4, seed=6, tag=f"small{s}")
                    for s, c in enumerate(ctx)])
    anc[1, 0] = 0
    run_packed(cfg, ctx, anc, "small")


def test_gpu_packed_bf16_head_dim64_odd_blocks():
    # head_dim 64, two query heads per KV head, block 10 and an odd number of
    # blocks per sequence (the last query tile holds one block); anchors at 0
    # and at the full context
    cfg = SMALL_BF16.with_(head_dim=64, n_kv_heads=4, block_size=10)
    ctx = [200, 333]
    anc = np.stack([I.training_anchors(c, 23, c // 4, seed=7, tag=f"hd64-{s}")
                    for s, c in enumerate(ctx)])
    anc[0, 0] = 0
    anc[1, -1] = ctx[1]
    run_packed(cfg, ctx, np.sort(anc, axis=1), "small-hd64")


def test_gpu_packed_anchor_past_context_is_clamped_and_flagged():
    run_packed(TINY_FP32, [32], [[5, 33]], "tiny-clamp", expect_flag=True)


def test_gpu_packed_qwen3_8b_shaped_sampled():
    cfg = QWEN3_8B_SHAPED
    ctx = [2048, 1500]
    nb = 128
    anc = np.stack([I.training_anchors(c, nb, 256, seed=6, tag=f"q8b{s}") for s, c in enumerate(ctx)])
    run_packed(cfg, ctx, anc, "q8b", layers=[0, cfg.n_layers - 1], sample=[0, 1, 63, 64, 126, 127])
