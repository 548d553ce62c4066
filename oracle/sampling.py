"""CPU oracle for temperature > 0 drafting and verification -- TEST
INFRASTRUCTURE, NOT PRODUCT CODE.

Only the tests, the package's smoke entry point and the benchmark's CPU leg
may import this module; the HIP library never imports, links or calls it, and
nothing here comes from the HIP side.

What is computed, with the passage it follows:

  [R] "DFlash: Why a Diffusion Drafter Can Accelerate an Autoregressive Model"
      (technical review), sec. 4.2, eqs. 6-8 and its Algorithm 1: draw each
      candidate from the draft's proposal law q, scan positions left to right,
      accept candidate y with probability min(1, p(y)/q(y)) (eq. 6); at the
      first rejection emit a sample of the residual law [p - q]_+ / Z (eq. 7);
      if every candidate survives, emit a bonus token from the target.
  [W] "DFlash: Block Diffusion for Flash Speculative Decoding" (wikillm
      summary), "Paper vs code": above temperature 0 the code uses this
      speculative rejection sampling with residual resampling.

Readings taken where the pages are silent (each repeated at its use):
  * p and q are the softmax of the target's and the draft's logits divided by
    the same temperature T > 0; top-p / top-k filtering is not applied.
  * the bonus token (all B-1 candidates accepted) is sampled from the target's
    law at the position after the last candidate (target row B-1 of B rows).
  * an empty residual support (p <= q everywhere, which eq. 7 makes a
    probability-0 event but rounding can reach) falls back to sampling p.
  * the random numbers are drawn from Philox4x32-10 (the counter-based
    generator of Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
    easy as 1, 2, 3", SC 2011), so the GPU side can draw the same numbers from
    the same published definition: key (low, high 32 bits of the 64-bit
    seed); counter (i // 4, row, round, stream), each below 2^32, with word
    i % 4; a uniform is ((w >> 9) + 0.5) / 2^23, exact in fp32 and fp64 (24
    significant bits). Streams: 0 drafting (row = draft row), 1 acceptance
    uniforms (row = sequence, i = position), 2 residual / bonus draws
    (row = sequence * B + position).
  * a categorical sample uses the Gumbel-max construction: the argmax of
    log-probability + (-log(-log u)) over the support is distributed as the
    law (a standard identity; pinned here by Monte Carlo), lowest index on ties.

Parity status: Philox is pinned to the generator's published known-answer
vectors (tests/golden/philox4x32_10_kat.txt); the
categorical sampler and the verification rule are pinned by Monte Carlo
against the target law (eq. 8) and by closed forms (eq. 7's acceptance mass,
the temperature -> 0 limit reducing to the greedy rule).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint64(0x9E3779B9)
_W1 = np.uint64(0xBB67AE85)
_M32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def philox4x32(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds [Salmon et al. 2011, sec. 4]: each round
    multiplies words 0 and 2 by the two round multipliers (32 x 32 -> 64-bit
    products), exchanges the halves of the products with words 1 and 3 xor
    the round key, and the key is bumped by the two Weyl constants between
    rounds. Words are held in uint64 arrays of any broadcastable shape
    (values below 2^32, so the products are exact); returns the four output
    words."""
    c = [np.asarray(x, dtype=np.uint64) for x in (c0, c1, c2, c3)]
    k = [np.asarray(k0, dtype=np.uint64), np.asarray(k1, dtype=np.uint64)]
    for x in c + k:
        assert np.all(x <= _M32), "Philox4x32 words are 32-bit"
    for r in range(10):
        p0 = _M0 * c[0]
        p1 = _M1 * c[2]
        c = [(p1 >> _S32) ^ c[1] ^ k[0], p1 & _M32, (p0 >> _S32) ^ c[3] ^ k[1], p0 & _M32]
        if r < 9:
            k = [(k[0] + _W0) & _M32, (k[1] + _W1) & _M32]
    return c


def _key(seed: int):
    seed = int(seed) % (1 << 64)
    return np.uint64(seed & 0xFFFFFFFF), np.uint64(seed >> 32)


def _to_uniform(w):
    return ((w >> np.uint64(9)).astype(np.float64) + 0.5) / float(1 << 23)


def uniforms(seed: int, idx, row, rnd: int, stream: int) -> np.ndarray:
    """u in (0, 1) for element indices idx of (row, round, stream): word
    idx % 4 of Philox4x32-10 at counter (idx // 4, row, round, stream), key
    (low, high half of seed); u = ((w >> 9) + 0.5) / 2^23."""
    idx = np.asarray(idx, dtype=np.uint64)
    row = np.asarray(row, dtype=np.uint64)
    words = philox4x32(idx >> np.uint64(2), row, np.uint64(rnd), np.uint64(stream), *_key(seed))
    sel = (idx & np.uint64(3)).astype(np.int64)
    return _to_uniform(np.choose(sel, words))


def row_uniforms(seed: int, V: int, rows, rnd: int, stream: int) -> np.ndarray:
    """uniforms(seed, arange(V), row, rnd, stream) for every row in rows
    ([len(rows), V]), computing each Philox block once for its four elements."""
    rows = np.asarray(rows, dtype=np.uint64).reshape(-1, 1)
    nb = (V + 3) // 4
    words = philox4x32(np.arange(nb, dtype=np.uint64)[None, :], rows, np.uint64(rnd),
                       np.uint64(stream), *_key(seed))
    w = np.stack(words, axis=-1).reshape(rows.shape[0], nb * 4)[:, :V]
    return _to_uniform(w)


def gumbel(u: np.ndarray) -> np.ndarray:
    return -np.log(-np.log(u))


def log_softmax(logits: np.ndarray, temperature: float) -> np.ndarray:
    """log of the law softmax(logits / T) over the last axis (reading: p and q
    are both taken at temperature T)."""
    z = np.asarray(logits, dtype=np.float64) / temperature
    m = np.max(z, axis=-1, keepdims=True)
    return z - (m + np.log(np.sum(np.exp(z - m), axis=-1, keepdims=True)))


def gumbel_argmax(scores: np.ndarray, g: np.ndarray):
    """argmax of scores + g over the last axis (lowest index on ties), and the
    margin between the best and second-best perturbed score."""
    s = scores + g
    top = np.argmax(s, axis=-1)  # first occurrence: lowest index on ties
    best = np.take_along_axis(s, top[..., None], axis=-1)[..., 0]
    if s.shape[-1] == 1:
        return top.astype(np.int64), np.full(best.shape, np.inf)
    rest = s.copy()
    np.put_along_axis(rest, top[..., None], -np.inf, axis=-1)
    return top.astype(np.int64), best - np.max(rest, axis=-1)


@dataclass
class Drafted:
    tokens: np.ndarray   # [rows] sampled candidate ids
    logq: np.ndarray     # [rows] log q(token)
    margins: np.ndarray  # [rows] best minus second-best perturbed score


def sample_drafts(logits: np.ndarray, temperature: float, seed: int, rnd: int) -> Drafted:
    """Candidates drawn from the draft's proposal laws q = softmax(logits / T)
    [R Algorithm 1 steps 2-3]; row r uses stream 0 with row index r."""
    logits = np.asarray(logits, dtype=np.float64)
    rows, V = logits.shape
    lq = log_softmax(logits, temperature)
    g = gumbel(row_uniforms(seed, V, np.arange(rows), rnd, 0))
    tok, margin = gumbel_argmax(lq, g)
    return Drafted(tok, lq[np.arange(rows), tok], margin)


@dataclass
class Verified:
    accept_len: np.ndarray   # [batch] accepted candidates a
    out_token: np.ndarray    # [batch] correction (a < m) or bonus (a = m)
    u_margin: np.ndarray     # [batch, m] |u_i - alpha_i| at the scanned positions (inf after)
    g_margin: np.ndarray     # [batch] perturbed-score margin of the emitted draw
    alpha: np.ndarray        # [batch, m] acceptance probabilities min(1, p/q)
    scores: np.ndarray       # [batch, V] perturbed scores of the emitted draw (its argmax
                             # is out_token; -inf outside the residual's support)


def verify(drafts: np.ndarray, draft_logits: np.ndarray, target_logits: np.ndarray,
           temperature: float, seed: int, rnd: int) -> Verified:
    """Speculative verification with residual resampling [R sec. 4.2, eqs. 6-7,
    Algorithm 1 steps 5-8 and 10] for a batch: drafts [b, m], draft logits
    [b, m, V] (the laws the candidates were drawn from), target logits
    [b, m+1, V] (the target's laws at the m candidate positions and the one
    after them). Sequences are independent; positions are scanned left to
    right and nothing after the first rejection is used."""
    drafts = np.asarray(drafts, dtype=np.int64)
    b, m = drafts.shape
    B = m + 1
    V = draft_logits.shape[-1]
    lq = log_softmax(draft_logits, temperature)
    lp = log_softmax(target_logits, temperature)
    sidx = np.arange(b)
    # eq. 6: candidate i is accepted when u_i < min(1, p_i(y_i) / q_i(y_i))
    u = uniforms(seed, np.arange(m)[None, :], sidx[:, None], rnd, 1)
    lpy = np.take_along_axis(lp[:, :m], drafts[..., None], -1)[..., 0]
    lqy = np.take_along_axis(lq, drafts[..., None], -1)[..., 0]
    alpha = np.minimum(1.0, np.exp(lpy - lqy))
    rejected = u >= alpha
    # a = first rejected position, m if every candidate survived
    a = np.where(rejected.any(1), np.argmax(rejected, 1), m)
    um = np.where(np.arange(m)[None, :] <= a[:, None], np.abs(u - alpha), np.inf)
    g = gumbel(row_uniforms(seed, V, sidx * B + a, rnd, 2))
    lp_a = lp[sidx, a]                                  # target law at the emitted position
    lq_a = lq[sidx, np.minimum(a, m - 1)]
    d = np.exp(lp_a) - np.exp(lq_a)
    # eq. 7: residual law [p - q]_+ / Z (Z only normalises: the argmax of
    # log[p - q]_+ + Gumbel ignores it); empty support (rounding only) and the
    # bonus (a = m) sample the target's law
    has_res = (a < m) & np.any(d > 0, axis=1)
    score = np.where(has_res[:, None],
                     np.where(d > 0, np.log(np.where(d > 0, d, 1.0)), -np.inf), lp_a)
    tok, margin = gumbel_argmax(score, g)
    return Verified(a.astype(np.int64), tok, um, margin, alpha, score + g)
