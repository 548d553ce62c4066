"""Pins for the CPU oracle: checks against things other than the oracle itself.

Every ``check_*`` takes the oracle module ``O`` and raises AssertionError when
the oracle disagrees with the pinned fact. ``tests/test_oracle_pins.py`` runs
them on the real oracle; ``tests/test_oracle_mutations.py`` runs them on copies
with a planted mistake and requires at least one to fail.

What the pins compare against:
  * library routines (torch ``rms_norm``, ``silu``, ``scaled_dot_product_attention``,
    ``linear``) and an independent torch re-derivation of a draft layer;
  * closed forms (RoPE as complex multiplication, RMS of a normalised row);
  * brute force on tiny inputs (attention by explicit loops, acceptance by
    enumeration against ``os.path.commonprefix``);
  * invariants (block-position permutation without RoPE, position shift with
    RoPE, GQA vs repeated-KV MHA, append split, batch independence, B = 1
    decode, empty context);
  * numbers the pages print (tests/golden/accounting_pins.json).
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import independent_torch as IT
from synth.configs import DrafterConfig

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def micro_cfg(**kw) -> DrafterConfig:
    base = DrafterConfig(
        name="micro", hidden=32, n_heads=4, n_kv_heads=2, head_dim=8, n_layers=2,
        intermediate=48, n_target_feats=3, target_hidden=16, vocab=50, block_size=4,
        rms_eps=1e-6, rope_theta=100.0, dtype="fp32", tied_embeddings=False)
    return base.with_(**kw)


def micro_weights(cfg: DrafterConfig, seed: int = 0, std: float = 0.25) -> dict:
    """Random fp64 weights with non-unit gains (so that every gain is exercised)."""
    rng = np.random.default_rng(seed)
    d, hd = cfg.hidden, cfg.head_dim
    w = {"embed": rng.normal(0, 1.0, (cfg.vocab, d)),
         "lm_head": rng.normal(0, std, (cfg.vocab, d)),
         "fc": rng.normal(0, std, (d, cfg.concat_width)),
         "fc_norm": 1 + 0.2 * rng.normal(size=d),
         "final_norm": 1 + 0.2 * rng.normal(size=d)}
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        w[p + "in_norm"] = 1 + 0.2 * rng.normal(size=d)
        w[p + "wq"] = rng.normal(0, std, (cfg.q_dim, d))
        w[p + "wk"] = rng.normal(0, std, (cfg.kv_dim, d))
        w[p + "wv"] = rng.normal(0, std, (cfg.kv_dim, d))
        w[p + "q_norm"] = 1 + 0.2 * rng.normal(size=hd)
        w[p + "k_norm"] = 1 + 0.2 * rng.normal(size=hd)
        w[p + "wo"] = rng.normal(0, std, (d, cfg.q_dim))
        w[p + "post_norm"] = 1 + 0.2 * rng.normal(size=d)
        w[p + "w_gate"] = rng.normal(0, std, (cfg.intermediate, d))
        w[p + "w_up"] = rng.normal(0, std, (cfg.intermediate, d))
        w[p + "w_down"] = rng.normal(0, std, (d, cfg.intermediate))
    return w


def micro_cache(O, cfg, w, ctx_len: int, seed: int = 1, start: int = 0):
    rng = np.random.default_rng(seed)
    feats = [rng.normal(size=(ctx_len, cfg.target_hidden)) for _ in range(cfg.n_target_feats)]
    ctx = O.ctx_project(feats, w["fc"], w["fc_norm"], cfg.rms_eps)
    return O.prefill_cache(ctx, start, w, cfg), feats, ctx


def _close(a, b, rtol=1e-10, atol=1e-10, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    scale = np.max(np.abs(b)) if b.size else 0.0
    assert err <= atol + rtol * scale, f"{what}: max err {err:.3e} (scale {scale:.3e})"


# ---------------------------------------------------------------------------
def check_rms_norm(O):
    rng = np.random.default_rng(2)
    x = rng.normal(size=(5, 24)) * 3
    g = rng.normal(size=24)
    ref = F.rms_norm(IT.t(x), (24,), weight=IT.t(g), eps=1e-6).numpy()
    _close(O.rms_norm(x, g, 1e-6), ref, what="rms_norm vs torch")
    # closed form: with unit gain the output's mean square is ms / (ms + eps)
    y = O.rms_norm(x, np.ones(24), 1e-3)
    ms = np.mean(x * x, axis=-1)
    _close(np.mean(y * y, axis=-1), ms / (ms + 1e-3), what="rms closed form")
    _close(O.rms_norm(np.array([[3.0, 4.0]]), np.ones(2), 0.0),
           np.array([[3.0, 4.0]]) / math.sqrt(12.5), what="rms hand example")


def check_silu(O):
    x = np.linspace(-30, 30, 121)
    _close(O.silu(x), F.silu(IT.t(x)).numpy(), what="silu vs torch")
    assert O.silu(np.array([0.0]))[0] == 0.0
    _close(O.silu(np.array([1.0])), [1.0 / (1.0 + math.exp(-1.0))], what="silu(1)")


def check_rope(O):
    rng = np.random.default_rng(3)
    # hand example: hd 4, theta 100 -> frequencies 1 and 0.1; position 1
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    c1, s1, c2, s2 = math.cos(1), math.sin(1), math.cos(0.1), math.sin(0.1)
    want = [1 * c1 - 3 * s1, 2 * c2 - 4 * s2, 3 * c1 + 1 * s1, 4 * c2 + 2 * s2]
    _close(O.rope(x, np.array([1]), 100.0), [want], what="rope hand example")
    # complex-multiplication form at many positions, theta 1e4, hd 64
    x = rng.normal(size=(7, 64))
    pos = np.array([0, 1, 5, 31, 1000, 32767, 40000])
    want = IT.rope_complex(IT.t(x), torch.as_tensor(pos), 1e4).numpy()
    _close(O.rope(x, pos, 1e4), want, rtol=1e-12, what="rope vs complex form")
    # norm preserved; dot product depends on the position difference only
    _close(np.linalg.norm(O.rope(x, pos, 1e4), axis=-1), np.linalg.norm(x, axis=-1),
           what="rope norm")
    q, k = rng.normal(size=(1, 64)), rng.normal(size=(1, 64))
    dots = [(O.rope(q, np.array([p + 7]), 1e4) @ O.rope(k, np.array([p]), 1e4).T).item()
            for p in (0, 3, 100, 5000)]
    _close(dots, [dots[0]] * 4, rtol=1e-9, what="rope relative position")


def check_attention_vs_sdpa(O):
    rng = np.random.default_rng(4)
    for (B, hq, hkv, hd, c) in [(4, 4, 2, 8, 7), (16, 8, 2, 16, 33), (3, 6, 6, 4, 0)]:
        q = rng.normal(size=(B, hq, hd))
        kb, vb = rng.normal(size=(B, hkv, hd)), rng.normal(size=(B, hkv, hd))
        kc, vc = rng.normal(size=(hkv, c, hd)), rng.normal(size=(hkv, c, hd))
        got = O.kv_injected_attention(q, kb, vb, kc, vc, hq // hkv)
        keys = torch.cat([IT.t(kc), IT.t(kb).transpose(0, 1)], dim=1)[None]
        vals = torch.cat([IT.t(vc), IT.t(vb).transpose(0, 1)], dim=1)[None]
        ref = F.scaled_dot_product_attention(IT.t(q).transpose(0, 1)[None], keys, vals,
                                             enable_gqa=True)[0].transpose(0, 1).numpy()
        _close(got, ref, what=f"attention vs sdpa {B, hq, hkv, hd, c}")


def check_attention_brute(O):
    rng = np.random.default_rng(5)
    B, hq, hkv, hd, c = 3, 4, 2, 4, 5
    q = rng.normal(size=(B, hq, hd))
    kb, vb = rng.normal(size=(B, hkv, hd)), rng.normal(size=(B, hkv, hd))
    kc, vc = rng.normal(size=(hkv, c, hd)), rng.normal(size=(hkv, c, hd))
    got = O.kv_injected_attention(q, kb, vb, kc, vc, hq // hkv)
    for i in range(B):
        for j in range(hq):
            g = j * hkv // hq
            keys = [kc[g, t] for t in range(c)] + [kb[t, g] for t in range(B)]
            vals = [vc[g, t] for t in range(c)] + [vb[t, g] for t in range(B)]
            sc = [sum(q[i, j, e] * kk[e] for e in range(hd)) / math.sqrt(hd) for kk in keys]
            ws = [math.exp(s) for s in sc]
            z = sum(ws)
            o = [sum(ws[t] * vals[t][e] for t in range(len(keys))) / z for e in range(hd)]
            _close(got[i, j], o, what=f"attention brute ({i},{j})")


def _window_mask(B, c, window):
    qpos = np.arange(c, c + B)[:, None]
    kpos = np.arange(c + B)[None, :]
    return torch.from_numpy(qpos - kpos < window)


def check_window_vs_sdpa_mask(O):
    # Sliding-window layers against torch SDPA with an explicit boolean mask:
    # query i (position c + i) sees key position p iff c + i - p < window.
    rng = np.random.default_rng(14)
    for (B, hq, hkv, hd, c, win) in [(4, 4, 2, 8, 20, 6), (4, 4, 2, 8, 20, 3), (16, 8, 2, 16, 40, 17),
                                     (5, 2, 1, 4, 9, 1), (4, 4, 2, 8, 7, 11), (3, 6, 6, 4, 0, 2)]:
        q = rng.normal(size=(B, hq, hd))
        kb, vb = rng.normal(size=(B, hkv, hd)), rng.normal(size=(B, hkv, hd))
        kc, vc = rng.normal(size=(hkv, c, hd)), rng.normal(size=(hkv, c, hd))
        got = O.kv_injected_attention(q, kb, vb, kc, vc, hq // hkv, win)
        keys = torch.cat([IT.t(kc), IT.t(kb).transpose(0, 1)], dim=1)[None]
        vals = torch.cat([IT.t(vc), IT.t(vb).transpose(0, 1)], dim=1)[None]
        ref = F.scaled_dot_product_attention(IT.t(q).transpose(0, 1)[None], keys, vals,
                                             attn_mask=_window_mask(B, c, win),
                                             enable_gqa=True)[0].transpose(0, 1).numpy()
        _close(got, ref, what=f"window attention vs sdpa {B, hq, hkv, hd, c, win}")


def check_window_hides_old_keys(O):
    # Context keys at positions p <= c - window are invisible to every query;
    # position c - window + 1 is visible to query 0 only.
    rng = np.random.default_rng(15)
    B, hq, hkv, hd, c, win = 4, 4, 2, 8, 12, 5
    q = rng.normal(size=(B, hq, hd))
    kb, vb = rng.normal(size=(B, hkv, hd)), rng.normal(size=(B, hkv, hd))
    kc, vc = rng.normal(size=(hkv, c, hd)), rng.normal(size=(hkv, c, hd))
    base = O.kv_injected_attention(q, kb, vb, kc, vc, hq // hkv, win)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, : c - win + 1] += 3.0
    vc2[:, : c - win + 1] -= 2.0
    _close(O.kv_injected_attention(q, kb, vb, kc2, vc2, hq // hkv, win), base,
           what="keys outside every query's window")
    kc3, vc3 = kc.copy(), vc.copy()
    vc3[:, c - win + 1] += 5.0
    moved = O.kv_injected_attention(q, kb, vb, kc3, vc3, hq // hkv, win)
    assert np.max(np.abs(moved[0] - base[0])) > 1e-6, "query 0 must see position c - window + 1"
    _close(moved[1:], base[1:], what="later queries must not see position c - window + 1")


def check_window_layers_in_forward(O):
    # Only the layers listed as sliding take the window: changing layer 1's
    # oldest context values changes the output when layer 1 is full-attention
    # and leaves it unchanged when layer 1 slides (window 3).
    cfg = micro_cfg(sliding_window=3, sliding_layers=(1,))
    w = micro_weights(cfg, seed=16)
    cache, _, _ = micro_cache(O, cfg, w, 10, seed=17)
    v1 = [x.copy() for x in cache.v]
    v1[1][:, :4] += 2.0
    moved = O.SeqCache(cache.k, v1)
    anchor = [3]
    full = cfg.with_(sliding_window=0, sliding_layers=())
    a = O.draft_forward(cfg, w, [cache], anchor).hidden
    b = O.draft_forward(cfg, w, [moved], anchor).hidden
    _close(b, a, what="sliding layer 1 ignores context outside its window")
    a = O.draft_forward(full, w, [cache], anchor).hidden
    b = O.draft_forward(full, w, [moved], anchor).hidden
    assert np.max(np.abs(a - b)) > 1e-6, "full-attention layer 1 must see every context row"
    # layer 0 is full attention in the sliding config too
    k0 = [x.copy() for x in cache.v]
    k0[0][:, :4] += 2.0
    a = O.draft_forward(cfg, w, [cache], anchor).hidden
    b = O.draft_forward(cfg, w, [O.SeqCache(cache.k, k0)], anchor).hidden
    assert np.max(np.abs(a - b)) > 1e-6, "layer 0 (not listed) must see every context row"


def check_wide_window_is_full_attention(O):
    rng = np.random.default_rng(18)
    B, hq, hkv, hd, c = 4, 4, 2, 8, 9
    q = rng.normal(size=(B, hq, hd))
    kb, vb = rng.normal(size=(B, hkv, hd)), rng.normal(size=(B, hkv, hd))
    kc, vc = rng.normal(size=(hkv, c, hd)), rng.normal(size=(hkv, c, hd))
    full = O.kv_injected_attention(q, kb, vb, kc, vc, hq // hkv)
    _close(O.kv_injected_attention(q, kb, vb, kc, vc, hq // hkv, c + B), full,
           what="window c + B = full attention")


def check_block_of_one_is_decode(O):
    """B = 1 (no mask tokens): the anchor's attention is the last row of a
    causal SDPA over [context ; anchor]; acceptance has nothing to accept."""
    rng = np.random.default_rng(6)
    hq, hkv, hd, c = 4, 2, 8, 9
    q = rng.normal(size=(1, hq, hd))
    kb, vb = rng.normal(size=(1, hkv, hd)), rng.normal(size=(1, hkv, hd))
    kc, vc = rng.normal(size=(hkv, c, hd)), rng.normal(size=(hkv, c, hd))
    got = O.kv_injected_attention(q, kb, vb, kc, vc, hq // hkv)
    keys = torch.cat([IT.t(kc), IT.t(kb).transpose(0, 1)], dim=1)[None]
    vals = torch.cat([IT.t(vc), IT.t(vb).transpose(0, 1)], dim=1)[None]
    qs = torch.cat([IT.t(rng.normal(size=(hq, c, hd))), IT.t(q).transpose(0, 1)], dim=1)[None]
    ref = F.scaled_dot_product_attention(qs, keys, vals, is_causal=True, enable_gqa=True)
    _close(got[0], ref[0, :, -1, :].numpy(), what="B=1 vs causal decode")
    acc, bonus = O.accept(np.zeros((3, 0), np.int64), np.array([[5], [7], [9]]))
    assert list(acc) == [0, 0, 0] and list(bonus) == [5, 7, 9], "B=1 accept"


def check_empty_context_is_block_mha(O):
    rng = np.random.default_rng(7)
    B, hq, hkv, hd = 5, 4, 4, 8
    q = rng.normal(size=(B, hq, hd))
    kb, vb = rng.normal(size=(B, hkv, hd)), rng.normal(size=(B, hkv, hd))
    empty = np.zeros((hkv, 0, hd))
    got = O.kv_injected_attention(q, kb, vb, empty, empty, 1)
    ref = F.scaled_dot_product_attention(IT.t(q).transpose(0, 1), IT.t(kb).transpose(0, 1),
                                         IT.t(vb).transpose(0, 1)).transpose(0, 1).numpy()
    _close(got, ref, what="empty context vs bidirectional MHA")


def check_ctx_project_and_kv_vs_torch(O):
    cfg = micro_cfg()
    w = micro_weights(cfg)
    rng = np.random.default_rng(8)
    feats = [rng.normal(size=(6, cfg.target_hidden)) for _ in range(cfg.n_target_feats)]
    ctx = O.ctx_project(feats, w["fc"], w["fc_norm"], cfg.rms_eps)
    _close(ctx, IT.ctx_project(feats, w["fc"], w["fc_norm"], cfg.rms_eps).numpy(),
           what="ctx_project vs torch")
    pos = np.arange(10, 16)
    cache = O.prefill_cache(ctx, 10, w, cfg)
    for l in range(cfg.n_layers):
        k, v = IT.context_kv(ctx, pos, O.layer_weights(w, l), cfg)
        _close(cache.k[l], k.numpy(), what=f"context K layer {l}")
        _close(cache.v[l], v.numpy(), what=f"context V layer {l}")


def check_draft_layer_vs_torch(O):
    for kw in ({}, {"n_kv_heads": 1}, {"block_size": 16, "head_dim": 16, "rope_theta": 1e4}):
        cfg = micro_cfg(**kw)
        w = micro_weights(cfg, seed=9)
        cache, _, _ = micro_cache(O, cfg, w, ctx_len=11)
        x = np.random.default_rng(10).normal(size=(cfg.block_size, cfg.hidden))
        for l in range(cfg.n_layers):
            lw = O.layer_weights(w, l)
            got = O.draft_layer(x, cache.k[l], cache.v[l], 11, lw, cfg)
            ref = IT.draft_layer(x, IT.t(cache.k[l]), IT.t(cache.v[l]), 11, lw, cfg).numpy()
            _close(got, ref, what=f"draft layer {l} vs torch {kw}")


def check_forward_structure(O):
    """Embedding of [anchor, MASK...], final norm, LM head on slots 1..B-1 and a
    lowest-index argmax, checked against torch on a micro drafter."""
    cfg = micro_cfg()
    w = micro_weights(cfg, seed=11)
    cache, _, _ = micro_cache(O, cfg, w, ctx_len=5)
    e = O.embed_block(7, w, cfg)
    _close(e[0], w["embed"][7], what="anchor row")
    for i in range(1, cfg.block_size):
        _close(e[i], w["embed"][cfg.mask_token_id], what="mask row")
    res = O.draft_forward(cfg, w, [cache], [7])
    x = e
    for l in range(cfg.n_layers):
        x = IT.draft_layer(x, IT.t(cache.k[l]), IT.t(cache.v[l]), 5, O.layer_weights(w, l), cfg)
    y = F.rms_norm(x[1:], (cfg.hidden,), weight=IT.t(w["final_norm"]), eps=cfg.rms_eps)
    logits = IT.lm_head(y, w["lm_head"]).numpy()
    _close(res.logits[0], logits, rtol=1e-9, what="forward logits vs torch")
    assert (res.drafts[0] == logits.argmax(-1)).all()
    srt = np.sort(logits, axis=-1)
    _close(res.margins[0], srt[:, -1] - srt[:, -2], what="margins")
    # tie-break: two equal maxima -> the lower id
    _, d, m = O.lm_head_argmax(np.array([[1.0, 0.0]]), np.array([[0.0, 0], [2, 0], [2, 0], [1, 0]]))
    assert int(d[0]) == 1 and m[0] == 0.0, "argmax tie-break"


def check_permutation_without_rope(O):
    cfg = micro_cfg(rope_theta=None, block_size=5)
    w = micro_weights(cfg, seed=12)
    cache, _, _ = micro_cache(O, cfg, w, ctx_len=6)
    x0 = np.random.default_rng(13).normal(size=(1, cfg.block_size, cfg.hidden))
    perm = np.array([3, 0, 4, 2, 1])
    a = O.draft_forward(cfg, w, [cache], [0], x0=x0)
    b = O.draft_forward(cfg, w, [cache], [0], x0=x0[:, perm])
    _close(b.hidden[0][:, :, :], a.hidden[0][:, perm, :], rtol=1e-9, what="permutation equivariance")


def check_position_shift_with_rope(O):
    cfg = micro_cfg(rope_theta=50.0)
    w = micro_weights(cfg, seed=14)
    rng = np.random.default_rng(15)
    feats = [rng.normal(size=(7, cfg.target_hidden)) for _ in range(cfg.n_target_feats)]
    ctx = O.ctx_project(feats, w["fc"], w["fc_norm"], cfg.rms_eps)
    a = O.draft_forward(cfg, w, [O.prefill_cache(ctx, 0, w, cfg)], [3])
    for shift in (1, 17, 123):
        b = O.draft_forward(cfg, w, [O.prefill_cache(ctx, shift, w, cfg)], [3],
                            start_pos=[7 + shift])
        _close(b.hidden, a.hidden, rtol=1e-9, what=f"position shift {shift}")
    c = O.draft_forward(cfg, w, [O.prefill_cache(ctx, 0, w, cfg)], [3], start_pos=[8])
    assert np.max(np.abs(c.hidden - a.hidden)) > 1e-6, "positions must matter with RoPE"


def check_gqa_equals_repeated_mha(O):
    cfg = micro_cfg(n_heads=4, n_kv_heads=2)
    w = micro_weights(cfg, seed=16)
    cache, _, _ = micro_cache(O, cfg, w, ctx_len=6)
    cfg2 = cfg.with_(n_kv_heads=4)
    w2 = dict(w)
    hd = cfg.head_dim
    rep = np.repeat(np.arange(cfg.n_kv_heads), cfg.group)
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        for name in ("wk", "wv"):
            w2[p + name] = w[p + name].reshape(cfg.n_kv_heads, hd, -1)[rep].reshape(-1, cfg.hidden)
    cache2 = O.SeqCache([k[rep] for k in cache.k], [v[rep] for v in cache.v])
    a = O.draft_forward(cfg, w, [cache], [1])
    b = O.draft_forward(cfg2, w2, [cache2], [1])
    _close(b.hidden, a.hidden, rtol=1e-10, what="GQA vs repeated-KV MHA")


def check_append_split(O):
    cfg = micro_cfg()
    w = micro_weights(cfg, seed=17)
    rng = np.random.default_rng(18)
    feats = [rng.normal(size=(9, cfg.target_hidden)) for _ in range(cfg.n_target_feats)]
    whole = O.prefill_cache(O.ctx_project(feats, w["fc"], w["fc_norm"], cfg.rms_eps), 0, w, cfg)
    parts = None
    for lo, hi in ((0, 4), (4, 5), (5, 9)):
        ctx = O.ctx_project([f[lo:hi] for f in feats], w["fc"], w["fc_norm"], cfg.rms_eps)
        c = O.prefill_cache(ctx, lo, w, cfg)
        parts = c if parts is None else parts.append(c)
    for l in range(cfg.n_layers):
        _close(parts.k[l], whole.k[l], what="append split K")
        _close(parts.v[l], whole.v[l], what="append split V")


def check_batch_independence(O):
    cfg = micro_cfg()
    w = micro_weights(cfg, seed=19)
    caches = [micro_cache(O, cfg, w, ctx_len=n, seed=20 + n)[0] for n in (3, 8, 1)]
    anchors = [4, 9, 13]
    batched = O.draft_forward(cfg, w, caches, anchors)
    for s in range(3):
        one = O.draft_forward(cfg, w, [caches[s]], [anchors[s]])
        _close(batched.hidden[s], one.hidden[0], rtol=1e-12, what=f"batch row {s}")
        _close(batched.logits[s], one.logits[0], rtol=1e-12, what=f"batch logits {s}")


def check_accept_bruteforce(O):
    for m in range(0, 4):
        for d in itertools.product(range(3), repeat=m):
            for tt in itertools.product(range(3), repeat=m + 1):
                acc, bonus = O.accept(np.array([d], dtype=np.int64).reshape(1, m),
                                      np.array([tt]))
                a = len(os.path.commonprefix([list(d), list(tt[:m])]))
                assert acc[0] == a and bonus[0] == tt[a], f"accept {d} {tt}"
    n_new, nxt = O.round_update(np.array([0, 3, 15]), np.array([11, 12, 13]))
    assert list(n_new) == [1, 4, 16] and list(nxt) == [11, 12, 13], "round update"


def check_select_layers(O):
    """Hand-worked cases (tests/golden/target_layer_selection.json), two with
    fractional points (halves round up, reading D12), plus properties that
    hold for any depth: first index 2 (layer 1, +1 offset), last L-2 (layer
    L-3, +1), strictly increasing, neighbouring gaps differing by at most 1."""
    with open(os.path.join(GOLDEN, "target_layer_selection.json")) as f:
        g = json.load(f)
    for e in g["cases"]:
        got = O.select_target_layers(e["n_target_layers"], e["n_feats"])
        assert got == e["ids"], (e, got)
    for L in range(8, 81):
        for n in (3, 5):
            ids = O.select_target_layers(L, n)
            gaps = np.diff(ids)
            assert len(ids) == n and ids[0] == 2 and ids[-1] == L - 2, (L, n, ids)
            assert (gaps > 0).all() and gaps.max() - gaps.min() <= 1, (L, n, ids)


def check_kv_cache_bytes(O):
    """[R sec. 5.3]'s cache-size formula against the bytes the library's cache
    layout actually allocates (K rows and 32-position V blocks, meta tensors,
    no memory touched) for the Qwen3-8B-shaped and tiny drafters."""
    import torch
    from block_diffusion_drafter_amd import binding as B
    for L, b, hkv, cap, hd, dt, es in ((5, 1, 8, 2048, 128, torch.bfloat16, 2),
                                       (5, 32, 8, 8192, 128, torch.bfloat16, 2),
                                       (1, 3, 2, 64, 64, torch.float32, 4)):
        c = B.KVCache(L, b, hkv, cap, hd, dt, device="meta")
        held = c.k.numel() * c.k.element_size() + c.v.numel() * c.v.element_size()
        assert O.kv_cache_bytes(b, L, cap, hkv * hd, es) == held, (L, b, cap, held)


def check_accounting(O):
    with open(os.path.join(GOLDEN, "accounting_pins.json")) as f:
        g = json.load(f)
    for e in g["tau_geometric"]:
        got = O.tau_geometric(e["a"], e["m"])
        assert abs(got - e["tau"]) <= e["abs_tol"], (e, got)
        tail = O.tau_tail_sum([e["a"] ** k for k in range(1, e["m"] + 1)])
        assert abs(tail - got) < 1e-12, "eq. 2 vs eq. 3"
    for e in g["cycle_speedup"]:
        got = O.cycle_speedup(e["tau"], e["r_d"], e["r_v"], e["r_o"])
        assert abs(got - e["speedup"]) <= e["abs_tol"], (e, got)
    for e in g["fusion_projection_bytes"]:
        assert O.fusion_projection_bytes(e["width"], e["n_feats"], e["bytes_per"]) == e["bytes"]
    for e in g["fusion_activation_bytes"]:
        inp, out = O.fusion_activation_bytes(e["n_tokens"], e["width"], e["n_feats"],
                                             e["bytes_per"])
        if "input_bytes_approx" in e:
            assert abs(inp / e["input_bytes_approx"] - 1) <= e["rel_tol"], inp
            assert abs(out / e["output_bytes_approx"] - 1) <= e["rel_tol"], out
        else:
            assert inp < e["input_bytes_below"], inp


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
