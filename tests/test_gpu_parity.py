"""HIP path vs the CPU oracle, element by element, through the C ABI.

Each test names its case before the first GPU call. Sizes are chosen so the
oracle finishes in seconds while the kernels still span several tiles and
ragged tails; the full-size Qwen3-8B-shaped case runs the whole prefill and
forward at batch 1, context 2048.
"""
import numpy as np
import pytest
import torch

from gpu_harness import (assert_close, assert_close_each, build_model, capacity_for,
                         check_accept, check_drafts, feats_to_device, log, prefix_offsets, to_np)
from block_diffusion_drafter_amd import binding as B
from oracle import dflash_oracle as O
from synth import QWEN3_8B_SHAPED, SMALL_BF16, TINY_FP32
from synth import inputs as I

pytestmark = pytest.mark.gpu


def test_gpu_accept_matches_oracle():
    log("case: accept, vocab 3, B in {1, 4, 16}")
    rng = np.random.default_rng(0)
    for Bk in (1, 4, 16):
        for b in (1, 7, 500):
            d = rng.integers(0, 3, size=(b, Bk - 1)).astype(np.int32)
            t = rng.integers(0, 3, size=(b, Bk)).astype(np.int32)
            t[: b // 2, : Bk - 1] = d[: b // 2]  # some full matches
            dg = torch.from_numpy(d).cuda()
            tg = torch.from_numpy(t).cuda()
            acc = torch.full((b,), -1, dtype=torch.int32, device="cuda")
            bon = torch.full((b,), -1, dtype=torch.int32, device="cuda")
            anc = torch.full((b,), -1, dtype=torch.int32, device="cuda")
            B.accept(dg, tg, Bk, acc, bon, anc)
            torch.cuda.synchronize()
            a_o, b_o = O.accept(d.astype(np.int64), t)
            assert (acc.cpu().numpy() == a_o).all()
            assert (bon.cpu().numpy() == b_o).all()
            assert (anc.cpu().numpy() == b_o).all()


def run_flow(cfg, ctx_lens, tag, seed=0, cap_extra=0, split_append=1, degenerate=False):
    """Prefill through ctx_project + ctx_kv_append, then one draft forward with
    fused accept on planted targets; every stage compared with the oracle.
    degenerate: the case's drafts are near ties by construction (e.g. every
    mask slot sees only mask slots), so the draft and accept checks run on the
    confident slots only, without requiring those to be the majority."""
    ctx_lens = [int(c) for c in ctx_lens]
    b, Bk, d = len(ctx_lens), cfg.block_size, cfg.hidden
    m = Bk - 1
    log(f"case: {cfg.name} batch {b} ctx {ctx_lens[:8]}{'...' if b > 8 else ''} ({tag})")
    M = build_model(cfg, seed)
    n_tot = sum(ctx_lens)
    cap = capacity_for(max(ctx_lens), Bk, cap_extra)
    feats = I.target_hiddens(cfg, n_tot, seed=1, tag=tag)
    dt = M.gpu.dtype
    ws = M.gpu.new_workspace(b, cap, max(n_tot, 1))
    ctx_gpu = torch.empty((max(n_tot, 1), d), dtype=dt, device="cuda")
    cache = M.gpu.new_cache(b, cap)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    if n_tot:
        M.gpu.ctx_project(feats_to_device(feats), ctx_gpu[:n_tot], ws)
    # append all rows, optionally over several calls that each take a slice of
    # every sequence's rows
    bounds = [np.linspace(0, c, split_append + 1).astype(int) for c in ctx_lens]
    cu_all = prefix_offsets(ctx_lens)
    for k in range(split_append):
        counts = [int(bounds[s][k + 1] - bounds[s][k]) for s in range(b)]
        rows = np.concatenate([np.arange(cu_all[s] + bounds[s][k], cu_all[s] + bounds[s][k + 1])
                               for s in range(b)]).astype(np.int64)
        part = ctx_gpu[torch.from_numpy(rows).cuda()] if len(rows) else ctx_gpu[:0]
        cu = torch.from_numpy(prefix_offsets(counts)).cuda()
        M.gpu.ctx_kv_append(cache, part.contiguous(), cu, ws, status)
    torch.cuda.synchronize()
    assert status.item() == 0, f"device status {status.item()}"
    assert cache.ctx_len.cpu().tolist() == ctx_lens

    ow = M.oracle_w
    ctx_o = O.ctx_project([f.f32() for f in feats], ow["fc"], ow["fc_norm"], cfg.rms_eps) \
        if n_tot else np.zeros((0, d))
    if n_tot:
        # per row: every context row is checked on its own
        assert_close(cfg, to_np(ctx_gpu[:n_tot]), ctx_o, "ctx_project", group_axes=1)
    caches = [O.prefill_cache(ctx_o[cu_all[s]:cu_all[s + 1]], 0, ow, cfg) for s in range(b)]
    for l in range(cfg.n_layers):
        # per sequence, grouped per KV head ([Hkv, n, hd])
        ks, vs = [], []
        for s in range(b):
            if not ctx_lens[s]:
                continue
            kg, vg = cache.read_positions(l, s, 0, ctx_lens[s])
            ks.append((f"seq {s}", to_np(kg), caches[s].k[l]))
            vs.append((f"seq {s}", to_np(vg), caches[s].v[l]))
        if ks:
            assert_close_each(cfg, ks, f"cache K layer {l}", group_axes=1)
            assert_close_each(cfg, vs, f"cache V layer {l}", group_axes=1)

    anchors = I.anchors(cfg, b, seed=3, tag=tag)
    res = O.draft_forward(cfg, ow, caches, anchors)
    a_star = I.planted_accept_lengths(b, m, seed=3, tag=tag)
    targets = I.plant_targets(res.drafts, a_star, cfg.vocab, seed=3, tag=tag)

    anchor_g = torch.from_numpy(anchors).cuda()
    drafts_g = torch.full((b, max(m, 1)), -1, dtype=torch.int32, device="cuda")
    logits_g = torch.empty((b, m, cfg.vocab), dtype=torch.float32, device="cuda")
    hidden_g = torch.empty((b, cfg.n_layers, Bk, d), dtype=torch.float32, device="cuda")
    tgt_g = torch.from_numpy(targets).cuda()
    acc_g = torch.full((b,), -1, dtype=torch.int32, device="cuda")
    bon_g = torch.full((b,), -1, dtype=torch.int32, device="cuda")
    M.gpu.draft_forward(cache, anchor_g, drafts_g, ws, logits=logits_g if m else None,
                        hidden_out=hidden_g, target_tokens=tgt_g, accept_len=acc_g,
                        bonus=bon_g, dev_status=status)
    torch.cuda.synchronize()
    assert status.item() == 0, f"device status {status.item()}"
    assert cache.ctx_len.cpu().tolist() == ctx_lens, "forward must not move ctx_len"
    for l in range(cfg.n_layers):
        assert_close(cfg, to_np(hidden_g[:, l]), res.hidden[:, l], f"hidden after layer {l}",
                     group_axes=1)
    drafts = drafts_g.cpu().numpy()[:, :m].astype(np.int64)
    if m:
        assert_close(cfg, to_np(logits_g), res.logits, "logits", group_axes=1)
        excl = check_drafts(res, drafts, "drafts", logits_g)
        if not degenerate:
            assert excl <= max(2, 0.5 * res.drafts.size), "too many low-margin slots to be a test"
    check_accept(res, targets, acc_g.cpu().numpy(), bon_g.cpu().numpy(), drafts, "accept")
    return M, cache, res


def test_gpu_tiny_fp32_end_to_end():
    run_flow(TINY_FP32, [32], "tiny")


def test_gpu_small_bf16_ragged_batch():
    # ragged contexts: empty, below one chunk, several chunks with a ragged tail
    run_flow(SMALL_BF16, [0, 37, 100, 301, 5], "small-ragged")


def test_gpu_small_bf16_split_append():
    run_flow(SMALL_BF16, [64, 129], "small-split", split_append=3)


def test_gpu_tiny_variants():
    # block of one (no mask slots), MHA (group 1), group 4 at head_dim 64 in fp32
    run_flow(TINY_FP32.with_(block_size=1), [32, 3], "tiny-b1")
    run_flow(TINY_FP32.with_(n_kv_heads=4), [20], "tiny-mha")
    run_flow(TINY_FP32.with_(n_heads=8, n_kv_heads=2), [45, 1], "tiny-g4")


def test_gpu_small_bf16_block8_two_layers():
    run_flow(SMALL_BF16.with_(block_size=8), [77, 200], "small-b8")


def test_gpu_small_bf16_gqa_groups_1_and_8():
    # bf16 attention with one query head per KV head (MHA) and with eight
    # (a KV group of 8 waves sharing each LDS block), contexts spanning one
    # and several workgroup ranges
    run_flow(SMALL_BF16.with_(n_kv_heads=8), [40, 900], "small-mha")
    run_flow(SMALL_BF16.with_(n_heads=16, n_kv_heads=2), [700, 33], "small-g8")


def test_gpu_small_bf16_batch1_hidden480():
    # One 16-row tile: the norms between projections are deferred to the
    # consumer; hidden 480 leaves 30 column tiles, so the consumer's float4
    # reads of the per-tile sums end in a partly used group.
    run_flow(SMALL_BF16.with_(hidden=480), [150], "small-h480")


def test_gpu_qwen3_8b_shaped_batch1_ctx2048():
    run_flow(QWEN3_8B_SHAPED, [2048], "q1")


def test_gpu_qwen3_dims_batch18_96row_blocks():
    # Qwen3-8B-shaped projections (small vocabulary, short contexts) at batch
    # 18: 270 context rows project and append on 96-row blocks, and the 288
    # forward rows run O and down on 96-row blocks with K slices.
    ctx = [0, 13, 9, 20, 23, 10, 12, 6, 25, 25, 19, 16, 16, 18, 20, 17, 21, 0]
    assert sum(ctx) == 270
    run_flow(QWEN3_8B_SHAPED.with_(vocab=4096), ctx, "q-dims-b18")


def test_gpu_capacity_overflow_is_flagged_and_clamped():
    cfg = TINY_FP32
    log(f"case: capacity overflow, {cfg.name}")
    M = build_model(cfg)
    cap = 64
    cache = M.gpu.new_cache(2, cap)
    guard_k = torch.randn_like(cache.k[:, 1])
    guard_v = torch.randn_like(cache.v[:, 1])
    cache.k[:, 1] = guard_k
    cache.v[:, 1] = guard_v
    ws = M.gpu.new_workspace(1, cap, 80)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    n = 70  # more rows than the capacity
    ctx = torch.randn((n, cfg.hidden), device="cuda")
    cu = torch.tensor([0, n, n], dtype=torch.int32, device="cuda")
    M.gpu.ctx_kv_append(cache, ctx, cu, ws, status)
    torch.cuda.synchronize()
    assert status.item() & B.DEV_CAPACITY
    assert cache.ctx_len.cpu().tolist() == [cap, 0]
    assert torch.equal(cache.k[:, 1], guard_k) and torch.equal(cache.v[:, 1], guard_v)
    # a forward with ctx_len at capacity cannot stage its block: flagged, no spill
    status.zero_()
    drafts = torch.empty((1, cfg.block_size - 1), dtype=torch.int32, device="cuda")
    M.gpu.draft_forward(cache, torch.tensor([5], dtype=torch.int32, device="cuda"), drafts, ws,
                        dev_status=status)
    torch.cuda.synchronize()
    assert status.item() & B.DEV_CAPACITY
    assert torch.equal(cache.k[:, 1], guard_k) and torch.equal(cache.v[:, 1], guard_v)
    # out-of-range anchor is clamped and flagged
    status.zero_()
    cache.ctx_len.fill_(10)
    M.gpu.draft_forward(cache, torch.tensor([cfg.vocab + 5], dtype=torch.int32, device="cuda"),
                        drafts, ws, dev_status=status)
    torch.cuda.synchronize()
    assert status.item() == B.DEV_TOKEN


def test_gpu_append_of_zero_rows_keeps_lengths_and_checks_offsets():
    # n_tok = 0: no projection, no cache write, only the length bookkeeping
    # and the offset checks (the round's append when no row was accepted is
    # never empty, but a caller's split append may be).
    cfg = TINY_FP32
    log(f"case: append of zero rows, {cfg.name}")
    M = build_model(cfg)
    cap = 64
    cache = M.gpu.new_cache(3, cap)
    cache.ctx_len.copy_(torch.tensor([5, 0, 63], dtype=torch.int32))
    cache.k.normal_()
    cache.v.normal_()
    k0, v0 = cache.k.clone(), cache.v.clone()
    ws = M.gpu.new_workspace(3, cap, 16)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ctx = torch.empty((0, cfg.hidden), device="cuda")
    M.gpu.ctx_kv_append(cache, ctx, torch.zeros(4, dtype=torch.int32, device="cuda"), ws, status)
    torch.cuda.synchronize()
    assert status.item() == 0
    assert cache.ctx_len.cpu().tolist() == [5, 0, 63]
    assert torch.equal(cache.k, k0) and torch.equal(cache.v, v0)
    # offsets that do not end at n_tok = 0 are flagged; nothing is written
    bad = torch.tensor([0, 0, 2, 2], dtype=torch.int32, device="cuda")
    M.gpu.ctx_kv_append(cache, ctx, bad, ws, status)
    torch.cuda.synchronize()
    assert status.item() & B.DEV_OFFSETS
    assert torch.equal(cache.k, k0) and torch.equal(cache.v, v0)


def test_gpu_small_bf16_merged_segments_groups_and_head_dim64():
    # batch >= 8: sequences that span several workgroups' key ranges are
    # merged by the last workgroup to finish (no combine launch); GQA groups
    # 8, 1 and 4, and head_dim 64, with ragged contexts (empty, short, long)
    ctx = [700, 33, 0, 90, 5, 300, 12, 640, 128]
    run_flow(SMALL_BF16.with_(n_heads=16, n_kv_heads=2), ctx, "small-g8-b9")
    run_flow(SMALL_BF16.with_(n_kv_heads=8), ctx[:8], "small-mha-b8")
    run_flow(SMALL_BF16.with_(head_dim=64, n_heads=8, n_kv_heads=2), ctx + [47, 2000], "small-hd64-b11")
