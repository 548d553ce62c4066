"""Device-resident decoding rounds: the accepted-rows injection and a whole
round captured once as a HIP graph and replayed, through the C ABI.

* dflash_ctx_kv_append_accepted against the oracle: the anchor and accepted
  rows of every sequence's block enter its context at the right positions,
  rows past the accept length stay unwritten, ctx_len advances on the device;
* a round graph replayed R times against the oracle's trajectory (accept,
  fuse, inject, draft): between replays the host writes the next targets and
  block features into the graph's fixed buffers, as a target pass would, and
  writes the oracle's drafts over the GPU's (teacher forcing, after checking
  them) so both sides follow one trajectory;
* graph replays against the same four calls made one by one on an identical
  state, bit for bit, over several replays with no host intervention in the
  device-resident state.
"""
import numpy as np
import pytest
import torch

from gpu_harness import (assert_close, assert_close_each, build_model, capacity_for,
                         check_drafts, feats_to_device, log,
                         prefix_offsets, to_np)
from block_diffusion_drafter_amd import binding as B
from oracle import dflash_oracle as O
from synth import SMALL_BF16, TINY_FP32
from synth import inputs as I

pytestmark = pytest.mark.gpu


def prefill(M, cfg, ctx_lens, tag, cap):
    """Prefill through ctx_project + ctx_kv_append on the GPU; the oracle's
    caches from the same features."""
    b, d = len(ctx_lens), cfg.hidden
    n_tot = int(sum(ctx_lens))
    feats = I.target_hiddens(cfg, n_tot, seed=1, tag=tag)
    ws = M.gpu.new_workspace(b, cap, max(n_tot, b * cfg.block_size))
    cache = M.gpu.new_cache(b, cap)
    ctx = torch.empty((n_tot, d), dtype=M.gpu.dtype, device="cuda")
    M.gpu.ctx_project(feats_to_device(feats), ctx, ws)
    M.gpu.ctx_kv_append(cache, ctx, torch.from_numpy(prefix_offsets(ctx_lens)).cuda(), ws)
    ctx_o = O.ctx_project([f.f32() for f in feats], M.oracle_w["fc"], M.oracle_w["fc_norm"],
                          cfg.rms_eps)
    cu = prefix_offsets(ctx_lens)
    caches = [O.prefill_cache(ctx_o[cu[s]:cu[s + 1]], 0, M.oracle_w, cfg) for s in range(b)]
    return cache, caches, ws


def block_features(cfg, b, seed, tag):
    return I.target_hiddens(cfg, b * cfg.block_size, seed=seed, tag=tag)


def oracle_append_accepted(M, cfg, caches, feats, acc):
    """The oracle's caches after rows s*B .. s*B + acc[s] join sequence s."""
    Bk = cfg.block_size
    ctx_o = O.ctx_project([f.f32() for f in feats], M.oracle_w["fc"], M.oracle_w["fc_norm"],
                          cfg.rms_eps)
    out = []
    for s, c in enumerate(caches):
        rows = ctx_o[s * Bk: s * Bk + int(acc[s]) + 1]
        out.append(c.append(O.prefill_cache(rows, c.ctx_len, M.oracle_w, cfg)))
    return out


def compare_caches(cfg, cache, caches, what):
    """Every sequence's cached K and V of every layer, grouped per KV head."""
    for l in range(cfg.n_layers):
        ks, vs = [], []
        for s, c in enumerate(caches):
            if not c.ctx_len:
                continue
            kg, vg = cache.read_positions(l, s, 0, c.ctx_len)
            ks.append((f"seq {s}", to_np(kg), c.k[l]))
            vs.append((f"seq {s}", to_np(vg), c.v[l]))
        assert_close_each(cfg, ks, f"{what}: K layer {l}", group_axes=1)
        assert_close_each(cfg, vs, f"{what}: V layer {l}", group_axes=1)


@pytest.mark.parametrize("cfg", [TINY_FP32, SMALL_BF16], ids=lambda c: c.name)
def test_gpu_append_accepted_matches_oracle(cfg):
    ctx_lens = [20, 0, 45, 7]
    b, Bk = len(ctx_lens), cfg.block_size
    log(f"case: append_accepted {cfg.name} batch {b} ctx {ctx_lens}")
    M = build_model(cfg)
    cap = capacity_for(max(ctx_lens) + Bk, Bk)
    cache, caches, ws = prefill(M, cfg, ctx_lens, "acc-prefill", cap)
    # mark every slot past the context so unwritten rows can be recognised
    for s, c in enumerate(ctx_lens):
        fill = torch.full((cfg.n_kv_heads, cap - c, cfg.head_dim), 7.0, device="cuda")
        for l in range(cfg.n_layers):
            cache.write_positions(l, s, c, fill, fill)
    acc = np.array([0, Bk - 1, Bk // 2, 1], dtype=np.int32)
    feats = block_features(cfg, b, seed=5, tag="acc-block")
    ctx = torch.empty((b * Bk, cfg.hidden), dtype=M.gpu.dtype, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    M.gpu.ctx_project(feats_to_device(feats), ctx, ws)
    M.gpu.ctx_kv_append_accepted(cache, ctx, torch.from_numpy(acc).cuda(), ws, status)
    torch.cuda.synchronize()
    assert status.item() == 0
    new_len = [c + int(a) + 1 for c, a in zip(ctx_lens, acc)]
    assert cache.ctx_len.cpu().tolist() == new_len
    caches = oracle_append_accepted(M, cfg, caches, feats, acc)
    compare_caches(cfg, cache, caches, "after append")
    for s in range(b):
        k, v = cache.read_positions(0, s, new_len[s], cap - new_len[s])
        assert bool((k.float() == 7.0).all()) and bool((v.float() == 7.0).all()), \
            f"seq {s}: rows past the accept length were written"


def test_gpu_append_accepted_flags_out_of_range_lengths():
    cfg = TINY_FP32
    ctx_lens = [3, 9]
    b, Bk = len(ctx_lens), cfg.block_size
    log(f"case: append_accepted out-of-range lengths, {cfg.name}")
    M = build_model(cfg)
    cap = capacity_for(max(ctx_lens) + Bk, Bk)
    cache, _, ws = prefill(M, cfg, ctx_lens, "acc-range", cap)
    ctx = torch.zeros((b * Bk, cfg.hidden), dtype=M.gpu.dtype, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    M.gpu.ctx_kv_append_accepted(cache, ctx, torch.tensor([-2, Bk + 5], dtype=torch.int32,
                                                           device="cuda"), ws, status)
    torch.cuda.synchronize()
    assert status.item() & B.DEV_OFFSETS
    # clamped to [0, B-1]: one row and B rows
    assert cache.ctx_len.cpu().tolist() == [ctx_lens[0] + 1, ctx_lens[1] + Bk]


class RoundBuffers:
    """The fixed buffers a round graph points at."""

    def __init__(self, M, cfg, b, cap, anchors, want_logits):
        Bk, m = cfg.block_size, cfg.block_size - 1
        self.feats = [torch.empty((b * Bk, cfg.target_hidden), dtype=M.gpu.dtype, device="cuda")
                      for _ in range(cfg.n_target_feats)]
        self.targets = torch.zeros((b, Bk), dtype=torch.int32, device="cuda")
        self.drafts = torch.full((b, m), -1, dtype=torch.int32, device="cuda")
        self.acc = torch.full((b,), -1, dtype=torch.int32, device="cuda")
        self.anchor = torch.from_numpy(np.asarray(anchors, dtype=np.int32)).cuda()
        self.ctx = torch.empty((b * Bk, cfg.hidden), dtype=M.gpu.dtype, device="cuda")
        self.logits = (torch.empty((b, m, cfg.vocab), dtype=torch.float32, device="cuda")
                       if want_logits else None)
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.ws = M.gpu.new_workspace(b, cap, b * Bk)

    def load(self, feats, targets):
        for dst, f in zip(self.feats, feats_to_device(feats)):
            dst.copy_(f)
        self.targets.copy_(torch.from_numpy(targets))

    def graph(self, M, cache):
        return B.RoundGraph(M.gpu, cache, self.feats, self.targets, self.drafts, self.acc,
                            self.anchor, self.ctx, self.ws, self.logits, self.status)

    def eager_round(self, M, cache):
        """The four calls the graph holds, one by one."""
        B.accept(self.drafts, self.targets, M.cfg.block_size, self.acc, self.anchor)
        M.gpu.ctx_project(self.feats, self.ctx, self.ws)
        M.gpu.ctx_kv_append_accepted(cache, self.ctx, self.acc, self.ws, self.status)
        M.gpu.draft_forward(cache, self.anchor, self.drafts, self.ws, logits=self.logits,
                            dev_status=self.status)


def test_gpu_round_graph_follows_the_oracle_trajectory():
    cfg = TINY_FP32
    ctx_lens = [20, 33, 7]
    b, Bk, m = len(ctx_lens), cfg.block_size, cfg.block_size - 1
    rounds = 6
    log(f"case: round graph vs oracle, {cfg.name} batch {b} ctx {ctx_lens}, {rounds} rounds")
    M = build_model(cfg)
    cap = capacity_for(max(ctx_lens) + Bk * (rounds + 1), Bk)
    cache, caches, _ = prefill(M, cfg, ctx_lens, "graph-prefill", cap)
    anchors = I.anchors(cfg, b, seed=3, tag="graph")
    buf = RoundBuffers(M, cfg, b, cap, anchors, want_logits=True)
    # the first block: an ordinary forward on both sides
    M.gpu.draft_forward(cache, buf.anchor, buf.drafts, buf.ws, logits=buf.logits,
                        dev_status=buf.status)
    res = O.draft_forward(cfg, M.oracle_w, caches, anchors)
    # the profiler's events cannot live in a graph: capture is refused meanwhile
    B.profiler_start(16)
    try:
        with pytest.raises(B.DFlashError, match="-8"):
            buf.graph(M, cache)
    finally:
        B.profiler_stop()
        B.profiler_reset()
    g = buf.graph(M, cache)
    torch.cuda.synchronize()
    for r in range(rounds):
        drafts = buf.drafts.cpu().numpy().astype(np.int64)
        check_drafts(res, drafts, f"round {r}: drafts", buf.logits)
        assert_close(cfg, to_np(buf.logits), res.logits, f"round {r}: logits", group_axes=1)
        # the target pass of this block: planted accept lengths against the
        # oracle's drafts, fresh features at every block position
        a_star = I.planted_accept_lengths(b, m, seed=100 + r, tag="graph")
        targets = I.plant_targets(res.drafts, a_star, cfg.vocab, seed=100 + r, tag="graph")
        feats = block_features(cfg, b, seed=200 + r, tag="graph-block")
        buf.load(feats, targets)
        buf.drafts.copy_(torch.from_numpy(res.drafts.astype(np.int32)))  # teacher forcing
        g.replay()
        a_o, bonus_o = O.accept(res.drafts, targets)
        assert (a_o == a_star).all()
        caches = oracle_append_accepted(M, cfg, caches, feats, a_o)
        res = O.draft_forward(cfg, M.oracle_w, caches, bonus_o)
        torch.cuda.synchronize()
        assert buf.status.item() == 0, f"round {r}: device status {buf.status.item()}"
        assert buf.acc.cpu().numpy().tolist() == a_o.tolist(), f"round {r}: accept lengths"
        assert buf.anchor.cpu().numpy().tolist() == bonus_o.tolist(), f"round {r}: anchors"
        assert cache.ctx_len.cpu().tolist() == [c.ctx_len for c in caches], f"round {r}: ctx_len"
        log(f"  round {r}: accept {a_o.tolist()}, ctx {[c.ctx_len for c in caches]}")
    drafts = buf.drafts.cpu().numpy().astype(np.int64)
    check_drafts(res, drafts, f"after {rounds} rounds: drafts", buf.logits)
    compare_caches(cfg, cache, caches, f"after {rounds} rounds")
    g.close()


@pytest.mark.parametrize("cfg", [SMALL_BF16, TINY_FP32], ids=lambda c: c.name)
def test_gpu_round_graph_replays_equal_eager_rounds(cfg):
    ctx_lens = [40, 3, 130, 64, 17, 90, 1, 250, 33]
    b, Bk, m = len(ctx_lens), cfg.block_size, cfg.block_size - 1
    rounds = 5
    log(f"case: round graph vs eager rounds, {cfg.name} batch {b}, {rounds} replays")
    M = build_model(cfg)
    cap = capacity_for(max(ctx_lens) + Bk * (rounds + 1), Bk)
    anchors = I.anchors(cfg, b, seed=3, tag="eq")
    states = []
    for _ in range(2):
        cache, _, _ = prefill(M, cfg, ctx_lens, "eq-prefill", cap)
        buf = RoundBuffers(M, cfg, b, cap, anchors, want_logits=True)
        M.gpu.draft_forward(cache, buf.anchor, buf.drafts, buf.ws, logits=buf.logits,
                            dev_status=buf.status)
        states.append((cache, buf))
    (ce, be), (cg, bg) = states
    g = bg.graph(M, cg)
    for r in range(rounds):
        torch.cuda.synchronize()
        d = be.drafts.cpu().numpy()
        assert np.array_equal(d, bg.drafts.cpu().numpy()), f"round {r}: drafts"
        # targets planted against the current drafts (device state untouched)
        a_star = I.planted_accept_lengths(b, m, seed=300 + r, tag="eq")
        targets = I.plant_targets(d.astype(np.int64), a_star, cfg.vocab, seed=300 + r, tag="eq")
        feats = block_features(cfg, b, seed=400 + r, tag="eq-block")
        be.load(feats, targets)
        bg.load(feats, targets)
        be.eager_round(M, ce)
        g.replay()
        torch.cuda.synchronize()
        assert be.acc.cpu().numpy().tolist() == a_star.tolist()
        for name in ("acc", "anchor", "drafts", "logits", "status"):
            x, y = getattr(be, name), getattr(bg, name)
            assert torch.equal(x, y), f"round {r}: {name} differs between graph and eager"
        assert torch.equal(ce.ctx_len, cg.ctx_len), f"round {r}: ctx_len"
    for l in range(cfg.n_layers):
        for s in range(b):
            n = int(ce.ctx_len[s])
            ke, ve = ce.read_positions(l, s, 0, n)
            kg, vg = cg.read_positions(l, s, 0, n)
            assert torch.equal(ke, kg) and torch.equal(ve, vg), f"cache layer {l} seq {s}"
    assert be.status.item() == 0 and bg.status.item() == 0
    log(f"  {rounds} replays bit-identical to eager rounds; ctx {ce.ctx_len.cpu().tolist()}")
    g.close()
