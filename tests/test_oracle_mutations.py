"""Plant plausible mistakes in the CPU oracle and require a pin to catch each.

Each mutation replaces one oracle function (on the CPU, inside this process)
with a subtly wrong variant -- a dropped term, a wrong sign, a wrong index, a
transposed operand -- then runs every pin in tests/oracle_pins.py. A mutation
that no pin notices would mean the pins leave that part of the oracle free.
"""
import numpy as np
import pytest

import oracle_pins as P
from oracle import dflash_oracle as O

_orig = {n: getattr(O, n) for n in dir(O) if callable(getattr(O, n))}


def _rope_sign(x, positions, theta):
    return _orig["rope"](x, -np.asarray(positions), theta)


def _rope_interleaved(x, positions, theta):
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    perm = np.concatenate([np.arange(0, hd, 2), np.arange(1, hd, 2)])
    y = _orig["rope"](x[..., perm], positions, theta)
    out = np.empty_like(y)
    out[..., perm] = y
    return out


def _rope_freq_off_by_one(x, positions, theta):
    if theta is None:
        return _orig["rope"](x, positions, theta)
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    half = hd // 2
    inv = float(theta) ** (-(np.arange(half) + 1.0) * 2.0 / hd)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv
    c, s = np.cos(ang), np.sin(ang)
    return np.concatenate([x[..., :half] * c - x[..., half:] * s,
                           x[..., half:] * c + x[..., :half] * s], axis=-1)


def _rms_no_eps_mean_sum(x, gain, eps):
    x = np.asarray(x, dtype=np.float64)
    return np.asarray(gain) * x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def _rms_gain_dropped(x, gain, eps):
    return _orig["rms_norm"](x, np.ones_like(np.asarray(gain, dtype=np.float64)), eps)


def _silu_sign(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(x))


def _attn_no_scale(q, kb, vb, kc, vc, group, window=None):
    hd = q.shape[-1]
    return _orig["kv_injected_attention"](np.asarray(q) * np.sqrt(hd), kb, vb, kc, vc, group,
                                          window)


def _attn_wrong_group(q, kb, vb, kc, vc, group, window=None):
    B, hq, hd = q.shape
    hkv = kb.shape[1]
    out = np.empty((B, hq, hd))
    for j in range(hq):
        one = _orig["kv_injected_attention"](q[:, j:j + 1], kb[:, [j % hkv]], vb[:, [j % hkv]],
                                             kc[[j % hkv]], vc[[j % hkv]], 1, window)
        out[:, j] = one[:, 0]
    return out


def _attn_causal_block(q, kb, vb, kc, vc, group, window=None):
    B = q.shape[0]
    out = np.empty(q.shape)
    for i in range(B):
        out[i] = _orig["kv_injected_attention"](q[i:i + 1], kb[:i + 1], vb[:i + 1], kc, vc,
                                                group, window)[0]
    return out


def _attn_block_keys_dropped(q, kb, vb, kc, vc, group, window=None):
    if kc.shape[1] == 0:
        return _orig["kv_injected_attention"](q, kb, vb, kc, vc, group, window)
    return _orig["kv_injected_attention"](q, kb[:0], vb[:0], kc, vc, group, window)


def _layer_no_attn_residual(x, ck, cv, sp, lw, cfg, trace=None, window=None):
    lw2 = dict(lw)
    return _orig["draft_layer"](x, ck, cv, sp, lw2, cfg, trace, window) - np.asarray(x) * 0.5


def _layer_k_from_q_weights(x, ck, cv, sp, lw, cfg, trace=None, window=None):
    lw2 = dict(lw)
    lw2["k_norm"] = lw["q_norm"]
    return _orig["draft_layer"](x, ck, cv, sp, lw2, cfg, trace, window)


def _layer_mlp_swapped(x, ck, cv, sp, lw, cfg, trace=None, window=None):
    lw2 = dict(lw)
    lw2["w_gate"], lw2["w_up"] = lw["w_up"], lw["w_gate"]
    return _orig["draft_layer"](x, ck, cv, sp, lw2, cfg, trace, window)


def _ctx_concat_reversed(feats, w_fc, g_fc, eps):
    return _orig["ctx_project"](list(feats)[::-1], w_fc, g_fc, eps)


def _ctx_transposed_w(feats, w_fc, g_fc, eps):
    c = np.concatenate([np.asarray(f, dtype=np.float64) for f in feats], axis=1)
    w = np.asarray(w_fc, dtype=np.float64)
    u = c @ w.reshape(w.shape[1], w.shape[0])
    return _orig["rms_norm"](u, g_fc, eps)


def _context_kv_no_rope(ctx, positions, lw, cfg):
    return _orig["context_kv"](ctx, np.zeros_like(np.asarray(positions)), lw, cfg)


def _prefill_positions_from_zero(ctx, start_pos, weights, cfg):
    return _orig["prefill_cache"](ctx, 0, weights, cfg)


def _embed_anchor_last(anchor, weights, cfg):
    e = _orig["embed_block"](anchor, weights, cfg)
    return e[::-1].copy()


def _argmax_last_tie(y, w_lm):
    logits, d, m = _orig["lm_head_argmax"](y, w_lm)
    rev = logits[..., ::-1]
    return logits, logits.shape[-1] - 1 - np.argmax(rev, axis=-1), m


def _accept_counts_all_matches(drafts, targets):
    drafts, targets = np.asarray(drafts), np.asarray(targets)
    b, m = drafts.shape
    acc = (drafts == targets[:, :m]).sum(axis=1)
    return acc, targets[np.arange(b), acc]


def _accept_bonus_shifted(drafts, targets):
    acc, _ = _orig["accept"](drafts, targets)
    targets = np.asarray(targets)
    return acc, targets[np.arange(len(acc)), np.minimum(acc + 1, targets.shape[1] - 1)]


def _select_no_offset(n, k=5):
    return [i - 1 for i in _orig["select_target_layers"](n, k)]


def _select_half_even(n, k=5):
    # numpy's round-half-to-even instead of the half-up reading
    return [int(v) + 1 for v in np.round(np.linspace(1, n - 3, k))]


def _select_truncate(n, k=5):
    return [int(v) + 1 for v in np.linspace(1, n - 3, k)]


def _tau_missing_one(a, m):
    return _orig["tau_geometric"](a, m) - 1.0


def _window_off_by_one(q, kb, vb, kc, vc, group, window=None):
    return _orig["kv_injected_attention"](q, kb, vb, kc, vc, group,
                                          None if window is None else window + 1)


def _window_reversed(q, kb, vb, kc, vc, group, window=None):
    # the window measured from the keys' side: hides the block's later keys
    if window is None:
        return _orig["kv_injected_attention"](q, kb, vb, kc, vc, group)
    B, hq, hd = q.shape
    c = kc.shape[1]
    out = np.empty((B, hq, hd))
    for i in range(B):
        # query i keeps the keys p with p - (c + i) < window
        lim = c + i + window
        keys_k = np.concatenate([kc, np.transpose(kb, (1, 0, 2))], axis=1)[:, :lim]
        keys_v = np.concatenate([vc, np.transpose(vb, (1, 0, 2))], axis=1)[:, :lim]
        out[i] = _orig["kv_injected_attention"](q[i:i + 1], kb[:0], vb[:0], keys_k, keys_v,
                                                group)[0]
    return out


def _layer_window_ignored(cfg, l):
    return None


def _layer_window_every_layer(cfg, l):
    w = getattr(cfg, "sliding_window", 0) or 0
    return int(w) if w > 0 else None


MUTATIONS = {
    "window_off_by_one": ("kv_injected_attention", _window_off_by_one),
    "window_reversed": ("kv_injected_attention", _window_reversed),
    "layer_window_ignored": ("layer_window", _layer_window_ignored),
    "layer_window_every_layer": ("layer_window", _layer_window_every_layer),
    "rope_sign": ("rope", _rope_sign),
    "rope_interleaved_pairs": ("rope", _rope_interleaved),
    "rope_freq_index": ("rope", _rope_freq_off_by_one),
    "rms_sum_not_mean": ("rms_norm", _rms_no_eps_mean_sum),
    "rms_gain_dropped": ("rms_norm", _rms_gain_dropped),
    "silu_sign": ("silu", _silu_sign),
    "attn_no_scale": ("kv_injected_attention", _attn_no_scale),
    "attn_wrong_group": ("kv_injected_attention", _attn_wrong_group),
    "attn_causal_block": ("kv_injected_attention", _attn_causal_block),
    "attn_block_keys_dropped": ("kv_injected_attention", _attn_block_keys_dropped),
    "layer_residual_scaled": ("draft_layer", _layer_no_attn_residual),
    "layer_wrong_k_norm": ("draft_layer", _layer_k_from_q_weights),
    "layer_gate_up_swapped": ("draft_layer", _layer_mlp_swapped),
    "ctx_concat_reversed": ("ctx_project", _ctx_concat_reversed),
    "ctx_weight_transposed": ("ctx_project", _ctx_transposed_w),
    "context_kv_no_rope": ("context_kv", _context_kv_no_rope),
    "prefill_positions": ("prefill_cache", _prefill_positions_from_zero),
    "embed_anchor_last": ("embed_block", _embed_anchor_last),
    "argmax_last_tie": ("lm_head_argmax", _argmax_last_tie),
    "accept_counts_all": ("accept", _accept_counts_all_matches),
    "accept_bonus_shifted": ("accept", _accept_bonus_shifted),
    "select_no_offset": ("select_target_layers", _select_no_offset),
    "select_half_even": ("select_target_layers", _select_half_even),
    "select_truncate": ("select_target_layers", _select_truncate),
    "tau_missing_one": ("tau_geometric", _tau_missing_one),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    fn_name, bad = MUTATIONS[name]
    monkeypatch.setattr(O, fn_name, bad)
    caught = []
    for check in P.ALL_CHECKS:
        try:
            check(O)
        except (AssertionError, ValueError, IndexError) as e:  # noqa: PERF203
            caught.append(check.__name__)
    assert caught, f"no pin catches mutation {name}"
