"""HIP path vs the oracle at the full-size workloads.

* batch 32, ragged contexts 512-8192, accept lengths planted on 0..15 against
  the oracle's drafts, fused accept;
* batch 32, the round's 261 new rows over the ragged contexts: ctx_project and
  every sequence's and layer's appended K/V;
* batch 4 at 32768 context: 1-16 new rows per sequence fused and injected with
  ctx_project + ctx_kv_append, then the forward;
* LLaMA-3.1-8B-shaped batch 16, 64 consecutive rounds (append, forward,
  accept, anchor <- bonus), teacher-forced by the oracle on sequence 0; the
  oracle tracks every sequence's cache, and on rounds 0, 21, 42 and 63 every
  sequence's hidden states (after every layer), logits, drafts and accept
  lengths are compared with it.

The cached context these workloads start from is a seeded synthetic cache
state (keys N(0,1), values N(0, (0.02*sqrt(d))^2)) written into the cache with
the binding's layout helpers; both sides read those same values. Every other
tensor is computed independently by each side.
"""
import numpy as np
import pytest
import torch

from gpu_harness import (assert_close, assert_close_each, build_model, capacity_for,
                         check_accept, check_drafts, log, prefix_offsets, to_np)
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
        assert_close(cfg, to_np(hidden[:, l]), res.hidden[:, l], f"{what}: hidden after layer {l}",
                     group_axes=1)
    if logits is not None:
        assert_close(cfg, to_np(logits), res.logits, f"{what}: logits", group_axes=1)
    check_drafts(res, drafts, f"{what}: drafts", logits)
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
    assert checked >= W.batch // 2, f"only {checked}/{W.batch} accept lengths compared"


def test_gpu_qwen3_8b_shaped_batch32_append():
    """The batch-32 round's append: 261 new rows over 32 ragged sequences
    (the projections' 96-row blocks), every sequence and layer against the
    oracle. Only the positions matter here, so the cache starts empty of
    values with the workload's context lengths."""
    W = WORKLOADS["q32"]
    cfg = W.model
    ctx_lens = I.ctx_lengths(W)
    # the round's draw of 1..B new rows per sequence (261 in all)
    n_new = np.random.Generator(np.random.PCG64(W.seeds["round_base"])).integers(
        1, cfg.block_size + 1, size=W.batch).astype(np.int32)
    n_tok = int(n_new.sum())
    log(f"case: {W.name} append, {n_tok} new rows {n_new.tolist()}")
    M = build_model(cfg)
    cap = capacity_for(int(ctx_lens.max()) + int(n_new.max()), cfg.block_size)
    cache = M.gpu.new_cache(W.batch, cap)
    cache.ctx_len.copy_(torch.as_tensor(ctx_lens.astype(np.int32)))
    ws = M.gpu.new_workspace(W.batch, cap, n_tok)
    feats = I.target_hiddens(cfg, n_tok, seed=W.seeds["round_base"], tag="q32.append")
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
    assert_close(cfg, to_np(ctx), ctx_o, "q32: ctx_project of new rows", group_axes=1)
    ks, vs = [], []
    for s in range(W.batch):
        new = O.prefill_cache(ctx_o[cu[s]:cu[s + 1]], int(ctx_lens[s]), ow, cfg)
        for l in range(cfg.n_layers):
            kg, vg = cache.read_positions(l, s, int(ctx_lens[s]), int(n_new[s]))
            ks.append((f"seq {s} layer {l}", to_np(kg), new.k[l]))
            vs.append((f"seq {s} layer {l}", to_np(vg), new.v[l]))
    assert_close_each(cfg, ks, "q32: appended K", group_axes=1)
    assert_close_each(cfg, vs, "q32: appended V", group_axes=1)


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
    assert_close(cfg, to_np(ctx), ctx_o, "q4l: ctx_project of new rows", group_axes=1)
    ks, vs = [], []
    for s in range(W.batch):
        new = O.prefill_cache(ctx_o[cu[s]:cu[s + 1]], int(ctx_lens[s]), ow, cfg)
        for l in range(cfg.n_layers):
            kg, vg = cache.read_positions(l, s, int(ctx_lens[s]), int(n_new[s]))
            ks.append((f"seq {s} layer {l}", to_np(kg), new.k[l]))
            vs.append((f"seq {s} layer {l}", to_np(vg), new.v[l]))
        seqs[s] = seqs[s].append(new)
    # per sequence and layer, grouped per KV head
    assert_close_each(cfg, ks, "q4l: appended K", group_axes=1)
    assert_close_each(cfg, vs, "q4l: appended V", group_axes=1)
    anchors = I.anchors(cfg, W.batch, seed=W.seeds["targets"], tag="q4l")
    log("  oracle forward at 32K context")
    res = O.draft_forward(cfg, ow, seqs, anchors)
    a_star = I.planted_accept_lengths(W.batch, cfg.block_size - 1, W.seeds["targets"], "q4l")
    targets = I.plant_targets(res.drafts, a_star, cfg.vocab, W.seeds["targets"], "q4l")
    out = run_forward(M, cfg, cache, anchors, targets, ws)
    checked = compare_forward(cfg, res, *out, targets, "q4l")
    assert checked >= W.batch // 2, f"only {checked}/{W.batch} accept lengths compared"


class GrowCache:
    """The oracle's view of one sequence's cache across rounds: fp64 buffers of
    a fixed capacity per layer, rows written in place as rounds append (so 64
    rounds of appends do not recopy the whole context each round)."""

    def __init__(self, seq: O.SeqCache, cap: int):
        hkv, n, hd = seq.k[0].shape
        self.n = n
        self.k = [np.zeros((hkv, cap, hd)) for _ in seq.k]
        self.v = [np.zeros((hkv, cap, hd)) for _ in seq.v]
        for l in range(len(seq.k)):
            self.k[l][:, :n] = seq.k[l]
            self.v[l][:, :n] = seq.v[l]

    def view(self) -> O.SeqCache:
        return O.SeqCache([k[:, :self.n] for k in self.k], [v[:, :self.n] for v in self.v])

    def append(self, new: O.SeqCache) -> None:
        r = new.ctx_len
        for l in range(len(self.k)):
            self.k[l][:, self.n:self.n + r] = new.k[l]
            self.v[l][:, self.n:self.n + r] = new.v[l]
        self.n += r


def test_gpu_llama31_8b_shaped_batch16_64_rounds():
    W = WORKLOADS["l16"]
    cfg = W.model
    b, Bk, m = W.batch, cfg.block_size, cfg.block_size - 1
    ctx_lens = I.ctx_lengths(W)
    rounds = W.rounds
    full_rounds = sorted({0, rounds // 3, (2 * rounds) // 3, rounds - 1})
    log(f"case: {W.name}, ctx0 {ctx_lens.tolist()}, {rounds} rounds, every sequence compared "
        f"on rounds {full_rounds}")
    M = build_model(cfg)
    cap = capacity_for(int(ctx_lens.max()) + 16 * rounds, Bk)
    cache, seqs = load_cache_state(M, cfg, ctx_lens, cap, seed=W.seeds["hiddens"])
    ws = M.gpu.new_workspace(b, cap, 16 * b)
    # fp64 weights once: the oracle then runs each round without re-widening
    ow = {k: np.asarray(v, dtype=np.float64) for k, v in M.oracle_w.items()}
    oc = [GrowCache(sq, cap) for sq in seqs]
    del seqs
    anchors = I.anchors(cfg, b, seed=W.seeds["targets"], tag="l16")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    checked0 = full_checked = 0
    for r in range(rounds):
        seed_r = W.seeds["round_base"] + r
        full = r in full_rounds
        # the oracle drafts sequence 0 (every sequence on the full rounds, from
        # the same anchors and cached context as the GPU); sequence 0's targets
        # are planted against the oracle's drafts
        res = O.draft_forward(cfg, ow, [c.view() for c in (oc if full else oc[:1])],
                              anchors if full else anchors[:1])
        a0 = I.planted_accept_lengths(1, m, seed_r, "l16")
        tgt = I.uniform_tokens(cfg, (b, Bk), seed_r, "l16.targets")
        tgt[:1] = I.plant_targets(res.drafts[:1], a0, cfg.vocab, seed_r, "l16")
        drafts, logits, hidden, acc, bon = run_forward(M, cfg, cache, anchors, tgt, ws)
        if full:
            # every sequence: hidden after every layer, logits, drafts, accept
            checked = compare_forward(cfg, res, drafts, logits, hidden, acc, bon, tgt,
                                      f"round {r}")
            assert checked >= b // 2, f"round {r}: only {checked}/{b} accept lengths compared"
            full_checked += checked
            res0 = O.ForwardResult(res.hidden[:1], res.logits[:1], res.drafts[:1],
                                   res.margins[:1])
        else:
            res0 = res
            for l in (0, cfg.n_layers - 1):
                assert_close(cfg, to_np(hidden[0, l]), res0.hidden[0, l],
                             f"round {r}: seq 0 hidden after layer {l}")
            check_drafts(res0, drafts[:1], f"round {r}: seq 0 drafts", logits[:1])
            checked0 += check_accept(res0, tgt[:1], acc[:1], bon[:1], drafts[:1],
                                     f"round {r}: seq 0 accept")
            # every other sequence: the prefix rule on its own drafts
            for s in range(1, b):
                a_own, b_own = O.accept(drafts[s:s + 1], tgt[s:s + 1])
                assert acc[s] == a_own[0] and bon[s] == b_own[0], f"round {r} seq {s}: prefix rule"
        a_o, b_o = O.accept(res0.drafts, tgt[:1])
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
        ctx_o = O.ctx_project([f.f32() for f in feats], ow["fc"], ow["fc_norm"], cfg.rms_eps)
        for s in range(b):
            oc[s].append(O.prefill_cache(ctx_o[cu[s]:cu[s + 1]], oc[s].n, ow, cfg))
        anchors = bon.astype(np.int32).copy()
        anchors[0] = int(b_o[0])
        torch.cuda.synchronize()
        assert status.item() == 0, f"round {r}: device status {status.item()}"
        if r % 8 == 0:
            log(f"  round {r}: ctx0 {oc[0].n}, accept0 {int(a_o[0])}")
    assert cache.ctx_len.cpu().numpy().tolist() == [c.n for c in oc]
    log(f"  sequence 0: {checked0}/{rounds - len(full_rounds)} accept lengths compared; "
        f"all sequences on {len(full_rounds)} rounds: {full_checked}/{b * len(full_rounds)}")
    assert checked0 >= (rounds - len(full_rounds)) // 2
