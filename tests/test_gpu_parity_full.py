"""HIP path vs the oracle at the full-size workloads.

* batch 32, ragged contexts 512-8192, accept lengths planted on 0..15 against
  the oracle's drafts, fused accept;
* batch 4 at 32768 context: 1-16 new rows per sequence fused and injected with
  ctx_project + ctx_kv_append, then the forward;
* LLaMA-3.1-8B-shaped batch 16, 64 consecutive rounds (append, forward,
  accept, anchor <- bonus), teacher-forced by the oracle on sequence 0.

The cached context these workloads start from is a seeded synthetic cache
state (keys N(0,1), values N(0, (0.02*sqrt(d))^2)) written into the cache with
the binding's layout helpers; both sides read those same values. Every other
tensor is computed independently by each side.
"""
import numpy as np
import pytest
import torch

from gpu_harness import (MARGIN, assert_close, build_model, capacity_for, check_accept,
                         check_drafts, log, prefix_offsets, to_np)
from oracle import dflash_oracle as O
from synth import WORKLOADS
from synth import inputs as I
from synth import torch_io

pytestmark = pytest.mark.gpu


def load_cache_state(M, cfg, ctx_lens, cap, seed):
    """Seeded cache state on both sides: host SeqCaches for the oracle and the
    same bf16 values written into a fresh GPU cache."""
    st = I.cache_state(cfg, ctx_lens, seed)
    b = len(ctx_lens)
    cache = M.gpu.new_cache(b, cap)
    seqs = []
    for s in range(b):
        ks, vs = [], []
        for l in range(cfg.n_layers):
            k, v = st[l][s]
            cache.write_positions(l, s, 0, torch_io.to_device(k), torch_io.to_device(v))
            ks.append(k.f32())
            vs.append(v.f32())
        seqs.append(O.SeqCache(ks, vs))
    cache.ctx_len.copy_(torch.as_tensor(np.asarray(ctx_lens, dtype=np.int32)))
    torch.cuda.synchronize()
    return cache, seqs


def run_forward(M, cfg, cache, anchors, targets, ws, want_logits=True):
    b, m = len(anchors), cfg.block_size - 1
    drafts = torch.full((b, m), -1, dtype=torch.int32, device="cuda")
    logits = torch.empty((b, m, cfg.vocab), dtype=torch.float32, device="cuda") \
        if want_logits else None
    hidden = torch.empty((b, cfg.n_layers, cfg.block_size, cfg.hidden), dtype=torch.float32,
                         device="cuda")
    acc = torch.full((b,), -1, dtype=torch.int32, device="cuda")
    bon = torch.full((b,), -1, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    M.gpu.draft_forward(cache, torch.from_numpy(np.asarray(anchors, np.int32)).cuda(), drafts, ws,
                        logits=logits, hidden_out=hidden,
                        target_tokens=torch.from_numpy(targets).cuda(), accept_len=acc,
                        bonus=bon, dev_status=status)
    torch.cuda.synchronize()
    assert status.item() == 0, f"device status {status.item()}"
    return (drafts.cpu().numpy().astype(np.int64), logits, hidden, acc.cpu().numpy(),
            bon.cpu().numpy())


def compare_forward(cfg, res, drafts, logits, hidden, acc, bon, targets, what):
    for l in range(cfg.n_layers):
        assert_close(cfg, to_np(hidden[:, l]), res.hidden[:, l], f"{what}: hidden after layer {l}")
    if logits is not None:
        assert_close(cfg, to_np(logits), res.logits, f"{what}: logits")
    check_drafts(res, drafts, f"{what}: drafts")
    return check_accept(res, targets, acc, bon, drafts, f"{what}: accept")


def test_gpu_qwen3_8b_shaped_batch32_ragged_planted_accept():
    W = WORKLOADS["q32"]
    cfg = W.model
    ctx_lens = I.ctx_lengths(W)
    log(f"case: {W.name}, ctx sum {int(ctx_lens.sum())}, min {ctx_lens.min()} max {ctx_lens.max()}")
    M = build_model(cfg)
    cap = capacity_for(int(ctx_lens.max()), cfg.block_size)
    cache, seqs = load_cache_state(M, cfg, ctx_lens, cap, seed=W.seeds["hiddens"])
    ws = M.gpu.new_workspace(W.batch, cap, 1)
    anchors = I.anchors(cfg, W.batch, seed=W.seeds["targets"], tag="q32")
    log("  oracle forward, 32 sequences")
    res = O.draft_forward(cfg, M.oracle_w, seqs, anchors)
    a_star = I.planted_accept_lengths(W.batch, cfg.block_size - 1, W.seeds["targets"], "q32")
    targets = I.plant_targets(res.drafts, a_star, cfg.vocab, W.seeds["targets"], "q32")
    out = run_forward(M, cfg, cache, anchors, targets, ws)
    checked = compare_forward(cfg, res, *out, targets, "q32")
    assert checked >= 3, "too few sequences with confident margins to check accept lengths"


def test_gpu_qwen3_8b_shaped_batch4_ctx32768_append():
    W = WORKLOADS["q4l"]
    cfg = W.model
    ctx_lens = I.ctx_lengths(W)
    n_new = I.append_counts(W)
    log(f"case: {W.name}, ctx {ctx_lens.tolist()}, new rows {n_new.tolist()}")
    M = build_model(cfg)
    cap = capacity_for(int(ctx_lens.max()) + int(n_new.max()), cfg.block_size)
    cache, seqs = load_cache_state(M, cfg, ctx_lens, cap, seed=W.seeds["hiddens"])
    n_tok = int(n_new.sum())
    ws = M.gpu.new_workspace(W.batch, cap, n_tok)
    feats = I.target_hiddens(cfg, n_tok, seed=W.seeds["round_base"], tag="q4l")
    ctx = torch.empty((n_tok, cfg.hidden), dtype=M.gpu.dtype, device="cuda")
    M.gpu.ctx_project([torch_io.to_device(f) for f in feats], ctx, ws)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    cu = prefix_offsets(n_new)
    M.gpu.ctx_kv_append(cache, ctx, torch.from_numpy(cu).cuda(), ws, status)
    torch.cuda.synchronize()
    assert status.item() == 0
    assert cache.ctx_len.cpu().numpy().tolist() == (ctx_lens + n_new).tolist()

    ow = M.oracle_w
    ctx_o = O.ctx_project([f.f32() for f in feats], ow["fc"], ow["fc_norm"], cfg.rms_eps)
    assert_close(cfg, to_np(ctx), ctx_o, "q4l: ctx_project of new rows")
    for s in range(W.batch):
        new = O.prefill_cache(ctx_o[cu[s]:cu[s + 1]], int(ctx_lens[s]), ow, cfg)
        for l in range(cfg.n_layers):
            kg, vg = cache.read_positions(l, s, int(ctx_lens[s]), int(n_new[s]))
            assert_close(cfg, to_np(kg), new.k[l], f"q4l: appended K seq {s} layer {l}")
            assert_close(cfg, to_np(vg), new.v[l], f"q4l: appended V seq {s} layer {l}")
        seqs[s] = seqs[s].append(new)
    anchors = I.anchors(cfg, W.batch, seed=W.seeds["targets"], tag="q4l")
    log("  oracle forward at 32K context")
    res = O.draft_forward(cfg, ow, seqs, anchors)
    a_star = I.planted_accept_lengths(W.batch, cfg.block_size - 1, W.seeds["targets"], "q4l")
    targets = I.plant_targets(res.drafts, a_star, cfg.vocab, W.seeds["targets"], "q4l")
    out = run_forward(M, cfg, cache, anchors, targets, ws)
    compare_forward(cfg, res, *out, targets, "q4l")


def test_gpu_llama31_8b_shaped_batch16_64_rounds():
    W = WORKLOADS["l16"]
    cfg = W.model
    b, Bk, m = W.batch, cfg.block_size, cfg.block_size - 1
    ctx_lens = I.ctx_lengths(W)
    rounds = W.rounds
    log(f"case: {W.name}, ctx0 {ctx_lens.tolist()}, {rounds} rounds")
    M = build_model(cfg)
    cap = capacity_for(int(ctx_lens.max()) + 16 * rounds, Bk)
    cache, seqs = load_cache_state(M, cfg, ctx_lens, cap, seed=W.seeds["hiddens"])
    ws = M.gpu.new_workspace(b, cap, 16 * b)
    # fp64 weights once: the oracle then runs each round without re-widening
    ow = {k: np.asarray(v, dtype=np.float64) for k, v in M.oracle_w.items()}
    seq0 = seqs[0]
    anchors = I.anchors(cfg, b, seed=W.seeds["targets"], tag="l16")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    checked = confident_drafts = 0
    for r in range(rounds):
        seed_r = W.seeds["round_base"] + r
        # the oracle drafts sequence 0; its targets are planted against those drafts
        res0 = O.draft_forward(cfg, ow, [seq0], anchors[:1])
        a0 = I.planted_accept_lengths(1, m, seed_r, "l16")
        tgt = I.uniform_tokens(cfg, (b, Bk), seed_r, "l16.targets")
        tgt[:1] = I.plant_targets(res0.drafts, a0, cfg.vocab, seed_r, "l16")
        drafts, _, hidden, acc, bon = run_forward(M, cfg, cache, anchors, tgt, ws,
                                                  want_logits=False)
        # sequence 0 against the oracle; every sequence against the prefix rule
        for l in (0, cfg.n_layers - 1):
            assert_close(cfg, to_np(hidden[0, l]), res0.hidden[0, l],
                         f"round {r}: seq 0 hidden after layer {l}")
        ok = res0.margins[0] > MARGIN
        assert (drafts[0][ok] == res0.drafts[0][ok]).all(), f"round {r}: confident drafts differ"
        confident_drafts += int(ok.sum())
        a_o, b_o = O.accept(res0.drafts, tgt[:1])
        for s in range(b):
            a_own, b_own = O.accept(drafts[s:s + 1], tgt[s:s + 1])
            assert acc[s] == a_own[0] and bon[s] == b_own[0], f"round {r} seq {s}: prefix rule"
        if (res0.margins[0, :min(int(a_o[0]), m - 1) + 1] > MARGIN).all():
            assert acc[0] == a_o[0] and bon[0] == b_o[0], f"round {r}: accept {acc[0]} vs {a_o[0]}"
            checked += 1
        # teacher forcing: both sides append the oracle's a+1 rows for seq 0 and
        # the GPU's own a+1 rows for the others; anchors become the bonus tokens
        n_new = (acc + 1).astype(np.int32)
        n_new[0] = int(a_o[0]) + 1
        n_tok = int(n_new.sum())
        feats = I.target_hiddens(cfg, n_tok, seed=seed_r, tag="l16.rows")
        ctx = torch.empty((n_tok, cfg.hidden), dtype=M.gpu.dtype, device="cuda")
        M.gpu.ctx_project([torch_io.to_device(f) for f in feats], ctx, ws)
        cu = prefix_offsets(n_new)
        M.gpu.ctx_kv_append(cache, ctx, torch.from_numpy(cu).cuda(), ws, status)
        ctx_o = O.ctx_project([f.f32()[:n_new[0]] for f in feats], ow["fc"], ow["fc_norm"],
                              cfg.rms_eps)
        seq0 = seq0.append(O.prefill_cache(ctx_o, seq0.ctx_len, ow, cfg))
        anchors = bon.astype(np.int32).copy()
        anchors[0] = int(b_o[0])
        torch.cuda.synchronize()
        assert status.item() == 0, f"round {r}: device status {status.item()}"
        if r % 8 == 0:
            log(f"  round {r}: ctx0 {seq0.ctx_len}, accept0 {int(a_o[0])}")
    assert cache.ctx_len.cpu().numpy()[0] == seq0.ctx_len
    log(f"  {checked}/{rounds} rounds with a confident accept length checked; "
        f"{confident_drafts} confident drafts matched")
    assert checked >= rounds // 8
