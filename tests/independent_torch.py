"""An independent re-derivation of the drafter layer from torch library routines.

Used only as a pin for the oracle: it shares no code with ``oracle/`` and is
built from library primitives (``F.linear``, ``F.rms_norm``, ``F.silu``,
``F.scaled_dot_product_attention`` with ``enable_gqa``) plus a complex-number
form of the rotary embedding, all in float64 on the CPU. A plausible mistake in
the oracle (a dropped scale, a wrong sign, a transposed operand, a wrong head
mapping) makes the two disagree.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

T64 = torch.float64


def t(a) -> torch.Tensor:
    return torch.as_tensor(np.asarray(a, dtype=np.float64))


def rope_complex(x: torch.Tensor, pos: torch.Tensor, theta) -> torch.Tensor:
    """x [..., n, hd]: element i and element i + hd/2 form the complex number
    x_i + 1j * x_{i+hd/2}, multiplied by exp(1j * pos * theta^(-2i/hd))."""
    if theta is None:
        return x
    hd = x.shape[-1]
    h = hd // 2
    z = torch.complex(x[..., :h], x[..., h:])
    freqs = torch.pow(torch.tensor(float(theta), dtype=T64),
                      -torch.arange(h, dtype=T64) * 2.0 / hd)
    rot = torch.polar(torch.ones(pos.shape[0], h, dtype=T64), pos.to(T64)[:, None] * freqs)
    z = z * rot
    return torch.cat([z.real, z.imag], dim=-1)


def head_norm(x: torch.Tensor, gain: torch.Tensor, eps: float) -> torch.Tensor:
    return F.rms_norm(x, (x.shape[-1],), weight=gain, eps=eps)


def ctx_project(feats, w_fc, g_fc, eps):
    c = torch.cat([t(f) for f in feats], dim=1)
    return F.rms_norm(F.linear(c, t(w_fc)), (t(w_fc).shape[0],), weight=t(g_fc), eps=eps)


def context_kv(ctx, positions, lw, cfg):
    ctx = t(ctx)
    n = ctx.shape[0]
    k = F.linear(ctx, t(lw["wk"])).view(n, cfg.n_kv_heads, cfg.head_dim).transpose(0, 1)
    v = F.linear(ctx, t(lw["wv"])).view(n, cfg.n_kv_heads, cfg.head_dim).transpose(0, 1)
    k = rope_complex(head_norm(k, t(lw["k_norm"]), cfg.rms_eps),
                     torch.as_tensor(np.asarray(positions)), cfg.rope_theta)
    return k, v


def draft_layer(x, k_ctx, v_ctx, start_pos, lw, cfg):
    """x [B, d]; k_ctx, v_ctx [Hkv, c, hd]."""
    x = t(x)
    B = x.shape[0]
    hq, hkv, hd, eps = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps
    pos = torch.arange(start_pos, start_pos + B)
    h = F.rms_norm(x, (x.shape[-1],), weight=t(lw["in_norm"]), eps=eps)
    q = F.linear(h, t(lw["wq"])).view(B, hq, hd).transpose(0, 1)      # [Hq, B, hd]
    k = F.linear(h, t(lw["wk"])).view(B, hkv, hd).transpose(0, 1)     # [Hkv, B, hd]
    v = F.linear(h, t(lw["wv"])).view(B, hkv, hd).transpose(0, 1)
    q = rope_complex(head_norm(q, t(lw["q_norm"]), eps), pos, cfg.rope_theta)
    k = rope_complex(head_norm(k, t(lw["k_norm"]), eps), pos, cfg.rope_theta)
    keys = torch.cat([t(k_ctx), k], dim=1)
    vals = torch.cat([t(v_ctx), v], dim=1)
    o = F.scaled_dot_product_attention(q.unsqueeze(0), keys.unsqueeze(0), vals.unsqueeze(0),
                                       is_causal=False, enable_gqa=True)[0]
    x = x + F.linear(o.transpose(0, 1).reshape(B, hq * hd), t(lw["wo"]))
    h2 = F.rms_norm(x, (x.shape[-1],), weight=t(lw["post_norm"]), eps=eps)
    x = x + F.linear(F.silu(F.linear(h2, t(lw["w_gate"]))) * F.linear(h2, t(lw["w_up"])),
                     t(lw["w_down"]))
    return x


def lm_head(y, w_lm):
    return F.linear(t(y), t(w_lm))
