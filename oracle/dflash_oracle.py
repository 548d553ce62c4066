"""CPU oracle for one DFlash drafter pass -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.

Only the tests, the package's smoke entry point and the benchmark's CPU-baseline
leg may import this module. The HIP library never imports, links or calls it,
and this module imports nothing from the HIP side: the two share no code. The
only module both consume is ``synth`` (seeded random draws, no arithmetic of
the method).

Plain NumPy in float64: every input (fp32 values, or bf16 bit patterns widened
exactly) is upcast to fp64 and no intermediate is rounded (compute_dtype() can
switch the same steps to float32 for the CPU throughput baseline only). Each function states
the passage it follows. Pages cited, by title:

  [W] "DFlash: Block Diffusion for Flash Speculative Decoding" -- wikillm.com
      paper summary (sections "Method", "Paper vs code", "Pitfalls", and its two
      inference pseudocode blocks: the greedy decoding loop and the draft layer).
  [R] "DFlash: Why a Diffusion Drafter Can Accelerate an Autoregressive Model"
      -- technical review of the v2 PDF (sections 2.3, 3.1, 4.1, 5.1, 5.3;
      equations 2-5 and 9-11).
  [K] "D-Flash: The Secret Behind 3.5x LLM Inference Speedup with Diffusion
      Drafting" -- kongchang.com (section "System Architecture").
  [A] "DFlash" -- aiwiki.ai encyclopedia entry (section "Method").

Readings taken where the pages are silent (each is repeated at its use):
  * pre-norm layers: RMSNorm before attention and before the MLP, one final
    RMSNorm before the LM head; the MLP is SwiGLU, down(SiLU(gate) * up).
  * per-head q/k RMSNorm over head_dim with a learned gain, before RoPE; it is
    applied to block queries, block keys and context keys alike.
  * rotary embedding pairs element i with element i + head_dim/2 ("rotate
    half"), inverse frequency theta^(-2i/head_dim); the block's position i sits
    at ctx_len + i; context rows keep their absolute positions.
  * attention scale 1/sqrt(head_dim), no mask; query head j reads KV head
    j // (n_heads / n_kv_heads); no biases anywhere.
  * sliding-window layers (listed in the config): query i of the block, at
    position ctx_len + i, sees the keys at positions p with
    ctx_len + i - p < window, and no causal mask.
  * context rows are not normed again per layer (they are already RMS-normed
    by the fusion step).
  * argmax ties break to the lowest token id.
  * the accept rule compares the B-1 drafts with the first B-1 target tokens.

Parity status: every function here is pinned by tests that do not re-run its
own formulas (library routines, closed forms, brute force, invariants and the
pages' printed numbers); the composed multi-layer pass has no printed worked
example on the pages, so beyond those pins the whole pass is "parity unpinned".
"""
from __future__ import annotations

import contextlib
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np

F64 = np.float64
# The type every step computes in: float64 for parity. compute_dtype() lets
# the CPU throughput baseline time the same steps in float32; no parity
# result is ever taken in that mode.
_COMPUTE = [F64]


@contextlib.contextmanager
def compute_dtype(dtype):
    """Run the oracle's arithmetic in dtype inside the block (timing only)."""
    prev = _COMPUTE[0]
    _COMPUTE[0] = np.dtype(dtype).type
    try:
        yield
    finally:
        _COMPUTE[0] = prev


def _f64(a) -> np.ndarray:
    """a in the compute type (float64 unless compute_dtype says otherwise)."""
    return np.asarray(a, dtype=_COMPUTE[0])


# ---------------------------------------------------------------------------
# Target-layer selection  [W "Paper vs code", second bullet]
# ---------------------------------------------------------------------------
def select_target_layers(n_target_layers: int, n_feats: int = 5) -> List[int]:
    """Indices of the target layers whose hidden states feed the drafter.

    [W "Paper vs code"]: layers spaced evenly from index 1 to index L-3; the
    code adds one when indexing a hidden-state list whose entry 0 is the
    embedding output. Reading: the evenly spaced points are rounded to the
    nearest integer, halves up (7.5 -> 8; the pages do not say). Returned
    values are hidden-state-list indices (+1 offset).
    """
    lo, hi = 1, n_target_layers - 3
    pts = np.linspace(lo, hi, n_feats)
    return [int(np.floor(p + 0.5)) + 1 for p in pts]


# ---------------------------------------------------------------------------
# Elementwise pieces
# ---------------------------------------------------------------------------
def rms_norm(x, gain, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: gain * x / sqrt(mean(x^2) + eps).
    [W "Method" Inference step 1, app. A.3: linear map followed by RMS
    normalisation]; [R eq. 9]."""
    x = _f64(x)
    return _f64(gain) * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def silu(x) -> np.ndarray:
    """SiLU(x) = x * sigmoid(x)."""
    x = _f64(x)
    return x / (1.0 + np.exp(-x))


def rope(x, positions, theta: Optional[float]) -> np.ndarray:
    """Rotary embedding of the last axis of x[..., n, hd] at integer positions [n].

    [W "Paper vs code", KV injection bullet]: rotary embeddings are applied and
    context keys sit at their absolute token positions. Reading: pairs
    (i, i + hd/2) are rotated by angle p * theta^(-2i/hd). theta=None disables
    the rotation (used only by invariance checks).
    """
    x = _f64(x)
    if theta is None:
        return x
    hd = x.shape[-1]
    half = hd // 2
    inv_freq = float(theta) ** (-np.arange(half, dtype=F64) * 2.0 / hd)
    ang = _f64(positions)[:, None] * inv_freq[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def softmax_rows(s) -> np.ndarray:
    s = _f64(s)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# Step a1: target-context-feature fusion   [R eq. 9]; [W "Method" step 1]
# ---------------------------------------------------------------------------
def ctx_project(feats: Sequence[np.ndarray], w_fc, g_fc, eps: float) -> np.ndarray:
    """H_t = RMSNorm(W_c [H^(l1); ...; H^(ln)]) for every context row.

    feats: the selected target layers' hidden states, each [n, d_t], in layer
    order; they are concatenated along the feature axis ([n, n_feat*d_t]),
    mapped by W_c [d, n_feat*d_t] (no bias) and RMS-normalised with gain g_fc.
    """
    c = np.concatenate([_f64(f) for f in feats], axis=1)
    u = c @ _f64(w_fc).T
    return rms_norm(u, g_fc, eps)


# ---------------------------------------------------------------------------
# Step a2: per-layer context K/V   [R eq. 10]; [W "Method" step 2, "Paper vs code"]
# ---------------------------------------------------------------------------
def context_kv(ctx, positions, lw: Dict[str, np.ndarray], cfg) -> tuple:
    """Context entries of one draft layer: K = RoPE(headRMS(ctx W_k^T)),
    V = ctx W_v^T, each [n_kv_heads, n, head_dim].

    The layer's own key/value weights are applied to the fused context feature
    (the same W_k, W_v that the block uses) [R eq. 10; W "Paper vs code"].
    The rows are stored and reused by later rounds [W "Method" step 2].
    """
    ctx = _f64(ctx)
    n = ctx.shape[0]
    hkv, hd = cfg.n_kv_heads, cfg.head_dim
    k = (ctx @ _f64(lw["wk"]).T).reshape(n, hkv, hd)
    v = (ctx @ _f64(lw["wv"]).T).reshape(n, hkv, hd)
    k = rms_norm(k, lw["k_norm"], cfg.rms_eps)
    k = np.stack([rope(k[:, g, :], positions, cfg.rope_theta) for g in range(hkv)])
    v = np.transpose(v, (1, 0, 2))
    return k, v


@dataclass
class SeqCache:
    """One sequence's cached context K/V for every draft layer:
    k[l], v[l] of shape [n_kv_heads, ctx_len, head_dim]."""
    k: List[np.ndarray]
    v: List[np.ndarray]

    @property
    def ctx_len(self) -> int:
        return self.k[0].shape[1]

    def append(self, other: "SeqCache") -> "SeqCache":
        return SeqCache([np.concatenate([a, b], axis=1) for a, b in zip(self.k, other.k)],
                        [np.concatenate([a, b], axis=1) for a, b in zip(self.v, other.v)])


def layer_weights(weights: Dict[str, np.ndarray], l: int) -> Dict[str, np.ndarray]:
    p = f"layers.{l}."
    return {k[len(p):]: v for k, v in weights.items() if k.startswith(p)}


def prefill_cache(ctx, start_pos: int, weights: Dict[str, np.ndarray], cfg) -> SeqCache:
    """Context K/V for rows at absolute positions start_pos .. start_pos+n-1."""
    pos = np.arange(start_pos, start_pos + np.asarray(ctx).shape[0])
    ks, vs = [], []
    for l in range(cfg.n_layers):
        k, v = context_kv(ctx, pos, layer_weights(weights, l), cfg)
        ks.append(k)
        vs.append(v)
    return SeqCache(ks, vs)


# ---------------------------------------------------------------------------
# Steps a3-a11: the draft layers   [W draft-layer pseudocode, "Method" step 2-3]
# ---------------------------------------------------------------------------
def embed_block(anchor: int, weights, cfg) -> np.ndarray:
    """Block [anchor, MASK x (B-1)] embedded with the shared embedding table
    (input_embedding_scale 1.0) [W "Method" step 3, "Paper vs code"]."""
    ids = np.array([anchor] + [cfg.mask_token_id] * (cfg.block_size - 1))
    return _f64(np.asarray(weights["embed"])[ids])


def kv_injected_attention(q, k_blk, v_blk, k_ctx, v_ctx, group: int,
                          window: Optional[int] = None) -> np.ndarray:
    """Non-causal attention of the block queries over [context ; block] keys.

    q [B, Hq, hd]; k_blk, v_blk [B, Hkv, hd]; k_ctx, v_ctx [Hkv, c, hd].
    [W draft-layer pseudocode]: keys and values are the context entries
    concatenated with the block's own along the sequence; queries come from the
    block only; [W "Paper vs code"]: full-attention layers are non-causal.
    Reading: scale 1/sqrt(hd), no mask, query head j uses KV head j // group.

    window: a sliding-window layer ([W "Paper vs code", attention-pattern
    bullet: the code supports per-layer sliding-window attention, which the
    paper does not describe]). Reading: with context positions 0..c-1 and
    block position i at c + i, query i sees key position p iff
    (c + i) - p < window; no causal part (the drafter is non-causal).
    """
    B, hq, hd = q.shape
    c = k_ctx.shape[1]
    qpos = np.arange(c, c + B)[:, None]
    kpos = np.arange(c + B)[None, :]
    visible = np.ones((B, c + B), dtype=bool) if window is None else (qpos - kpos < window)
    out = np.empty((B, hq, hd), dtype=_COMPUTE[0])
    for j in range(hq):
        g = j // group
        keys = np.concatenate([_f64(k_ctx[g]), _f64(k_blk[:, g, :])], axis=0)
        vals = np.concatenate([_f64(v_ctx[g]), _f64(v_blk[:, g, :])], axis=0)
        scores = np.where(visible, _f64(q[:, j, :]) @ keys.T / np.sqrt(hd), -np.inf)
        p = softmax_rows(scores)
        out[:, j, :] = p @ vals
    return out


def layer_window(cfg, l: int) -> Optional[int]:
    """The attention window of draft layer l: the config's sliding_window for
    the layers listed in sliding_layers, None (full attention) otherwise."""
    w = getattr(cfg, "sliding_window", 0) or 0
    return int(w) if w > 0 and l in tuple(getattr(cfg, "sliding_layers", ())) else None


def draft_layer(x, cache_k, cache_v, start_pos: int, lw, cfg, trace: Optional[dict] = None,
                window: Optional[int] = None) -> np.ndarray:
    """One draft layer over one sequence's block x [B, d] (fp64 residual).

    [W draft-layer pseudocode]: queries from the block, keys/values from
    context and block, residual update of the block only, then the
    feed-forward block with its own residual. Readings: pre-norm RMSNorm before
    attention and MLP; SwiGLU MLP; per-head q/k RMSNorm then RoPE at positions
    start_pos + i.
    """
    B = x.shape[0]
    hq, hkv, hd, eps = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps
    pos = np.arange(start_pos, start_pos + B)
    h = rms_norm(x, lw["in_norm"], eps)
    q = (h @ _f64(lw["wq"]).T).reshape(B, hq, hd)
    k = (h @ _f64(lw["wk"]).T).reshape(B, hkv, hd)
    v = (h @ _f64(lw["wv"]).T).reshape(B, hkv, hd)
    q = rms_norm(q, lw["q_norm"], eps)
    k = rms_norm(k, lw["k_norm"], eps)
    q = np.stack([rope(q[:, j, :], pos, cfg.rope_theta) for j in range(hq)], axis=1)
    k = np.stack([rope(k[:, g, :], pos, cfg.rope_theta) for g in range(hkv)], axis=1)
    o = kv_injected_attention(q, k, v, cache_k, cache_v, hq // hkv, window)
    x = x + o.reshape(B, hq * hd) @ _f64(lw["wo"]).T
    h2 = rms_norm(x, lw["post_norm"], eps)
    act = silu(h2 @ _f64(lw["w_gate"]).T) * (h2 @ _f64(lw["w_up"]).T)
    x = x + act @ _f64(lw["w_down"]).T
    if trace is not None:
        trace.setdefault("q", []).append(q)
        trace.setdefault("k_blk", []).append(k)
        trace.setdefault("v_blk", []).append(v)
        trace.setdefault("attn", []).append(o)
    return x


@dataclass
class ForwardResult:
    hidden: np.ndarray      # [b, n_layers, B, d] residual stream after each layer
    logits: np.ndarray      # [b, B-1, V]
    drafts: np.ndarray      # [b, B-1] int
    margins: np.ndarray     # [b, B-1] top1 - top2 logit


def lm_head_argmax(y, w_lm):
    """Logits = y W_lm^T (output_multiplier 1.0, no soft-cap), greedy argmax with
    the lowest id on ties, and the top-1 minus top-2 margin.
    [W "Paper vs code": drafted tokens bullet; decoding-loop pseudocode]."""
    logits = _f64(y) @ _f64(w_lm).T
    drafts = np.argmax(logits, axis=-1)
    top2 = np.partition(logits, -2, axis=-1)[..., -2:]
    margins = top2[..., 1] - top2[..., 0]
    return logits, drafts, margins


def draft_forward(cfg, weights: Dict[str, np.ndarray], caches: Sequence[SeqCache],
                  anchors: Sequence[int], start_pos: Optional[Sequence[int]] = None,
                  x0: Optional[np.ndarray] = None, trace: Optional[dict] = None
                  ) -> ForwardResult:
    """One parallel drafter pass for a batch of sequences.

    [W decoding-loop pseudocode]: embed [anchor] + [MASK]*(B-1), run the
    drafter over it with the context, apply the shared LM head to every output
    but the anchor's, and take the argmax. Each sequence attends only to its own
    cache; rows of different sequences never mix. ``start_pos`` overrides the
    block's first position (default: the sequence's context length); ``x0``
    [b, B, d] overrides the embedded block (invariance checks only).
    """
    b = len(caches)
    B, d = cfg.block_size, cfg.hidden
    xs = np.stack([embed_block(int(anchors[s]), weights, cfg) if x0 is None else _f64(x0[s])
                   for s in range(b)])
    hidden = np.empty((b, cfg.n_layers, B, d), dtype=_COMPUTE[0])
    for l in range(cfg.n_layers):
        lw = layer_weights(weights, l)
        for s in range(b):
            sp = caches[s].ctx_len if start_pos is None else int(start_pos[s])
            xs[s] = draft_layer(xs[s], caches[s].k[l], caches[s].v[l], sp, lw, cfg,
                                trace=trace if s == 0 else None, window=layer_window(cfg, l))
            hidden[s, l] = xs[s]
    y = rms_norm(xs[:, 1:, :], weights["final_norm"], cfg.rms_eps)
    logits, drafts, margins = lm_head_argmax(y, weights["lm_head"])
    return ForwardResult(hidden, logits, drafts.astype(np.int64), margins)


# ---------------------------------------------------------------------------
# Steps a14-a15: greedy acceptance and round update
# ---------------------------------------------------------------------------
def accept(drafts, targets):
    """Greedy accept-prefix. [W decoding-loop pseudocode]: accepted = number of
    leading drafts equal to the target's tokens (the drafts are compared with
    posterior[:-1]); bonus = posterior[accepted]; [W "Paper vs code"]: the
    acceptance length tau counts the bonus (accepted + 1). [R sec. 4.1]: keep
    the longest agreeing prefix, then emit the target's own token.

    drafts [b, m], targets [b, m+1] -> (accepted [b], bonus [b])."""
    drafts = np.asarray(drafts)
    targets = np.asarray(targets)
    b, m = drafts.shape
    acc = np.zeros(b, dtype=np.int64)
    bonus = np.zeros(b, dtype=np.int64)
    for s in range(b):
        a = 0
        while a < m and drafts[s, a] == targets[s, a]:
            a += 1
        acc[s] = a
        bonus[s] = targets[s, a]
    return acc, bonus


def round_update(accepted, bonus):
    """[W decoding-loop pseudocode]: the context grows by the verified features
    of [anchor + accepted drafts] (accepted + 1 rows) and the next anchor is the
    bonus token. Returns (rows to append [b], next anchor [b])."""
    return np.asarray(accepted) + 1, np.asarray(bonus)


# ---------------------------------------------------------------------------
# Accounting helpers that the pages print numbers for
# ---------------------------------------------------------------------------
def tau_tail_sum(p_at_least: Sequence[float]) -> float:
    """[R eq. 2]: tau = E[A+1] = 1 + sum_{k=1..m} Pr(A >= k)."""
    return 1.0 + float(np.sum(_f64(p_at_least)))


def tau_geometric(a: float, m: int) -> float:
    """[R eq. 3]: with a constant per-token survival a, Pr(A >= k) = a^k and
    tau = (1 - a^(m+1)) / (1 - a)."""
    return (1.0 - a ** (m + 1)) / (1.0 - a)


def cycle_speedup(tau: float, r_d: float, r_v: float, r_o: float = 0.0) -> float:
    """[R eqs. 4-5]: S = tau * L_t / (T_d + T_v + T_o) = tau / (r_d + r_v + r_o)
    with costs normalised by the autoregressive per-token time; [W eq. 1] is the
    r_o = 0 case."""
    return tau / (r_d + r_v + r_o)


def fusion_projection_bytes(width: int, n_feats: int, bytes_per: int) -> int:
    """[R eq. 11]: weights of the fusion projection, n_feats*width inputs to
    width outputs."""
    return n_feats * width * width * bytes_per


def fusion_activation_bytes(n_tokens: int, width: int, n_feats: int, bytes_per: int) -> tuple:
    """[R sec. 5.3]: concatenated fusion input and projected output sizes for
    n_tokens context rows."""
    return n_tokens * n_feats * width * bytes_per, n_tokens * width * bytes_per


def kv_cache_bytes(batch: int, n_layers: int, ctx_tokens: int, d_kv: int, bytes_per: int) -> int:
    """[R sec. 5.3]: rough draft-side context cache size 2*b*d*L*d_kv*s."""
    return 2 * batch * n_layers * ctx_tokens * d_kv * bytes_per
