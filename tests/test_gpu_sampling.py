"""Temperature > 0 drafting and verification: the HIP kernels against the
oracle (oracle/sampling.py) on the same seeded fp32 logits and the same
Philox4x32-10 random numbers (each side implements the generator from its
published definition).

Decisions are compared bit-exactly wherever floating point cannot decide them
differently: a sampled token where the oracle's best-minus-second perturbed
score exceeds 1e-3, an acceptance test where |u - alpha| exceeds 1e-4 (fp32
on the GPU against fp64 in the oracle). Below those margins several answers
are correct, and the GPU's is checked to be one of them: a sampled token's
oracle perturbed score lies within 1e-3 of the best, and an accept length
that differs from the oracle's flips at a position where |u - alpha| is
within 1e-4. Everything else holds at any margin (ranges, the accept-all case
p = q).
"""
import numpy as np
import pytest
import torch

from block_diffusion_drafter_amd import binding as B
from gpu_harness import log
from oracle import sampling as S
from synth import inputs as I

pytestmark = pytest.mark.gpu

G_MARGIN = 1e-3
U_MARGIN = 1e-4


def logits(shape, seed, name, std):
    return I.normal(seed, name, shape, std, False).reshape(shape)


@pytest.mark.parametrize("rows,V,T", [(45, 1000, 0.7), (30, 151936, 1.0), (7, 37, 1.5),
                                      (16, 8193, 0.9)])
def test_gpu_sample_drafts_matches_oracle(rows, V, T):
    log(f"case: sample_drafts rows {rows} vocab {V} T {T}")
    lg = logits((rows, V), 21, f"sample{V}", 2.0)
    ref = S.sample_drafts(lg, T, seed=123, rnd=4)
    tok = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    lq = torch.empty(rows, dtype=torch.float32, device="cuda")
    ws = B.sampling_workspace(rows, 2, V)
    B.sample_drafts(torch.from_numpy(lg).cuda(), T, 123, 4, tok, ws, lq)
    torch.cuda.synchronize()
    tok = tok.cpu().numpy()
    lq = lq.cpu().numpy().astype(np.float64)
    assert ((tok >= 0) & (tok < V)).all()
    ok = ref.margins > G_MARGIN
    assert (tok[ok] == ref.tokens[ok]).all(), np.argwhere((tok != ref.tokens) & ok)[:5]
    assert (~ok).sum() <= max(1, rows // 10)
    # every row, near-ties included: the GPU's token is within G_MARGIN of the
    # oracle's best perturbed score (log q + Gumbel noise of the same Philox draws)
    score = S.log_softmax(lg, T) + S.gumbel(S.row_uniforms(123, V, np.arange(rows), 4, 0))
    gap = score.max(axis=1) - score[np.arange(rows), tok]
    assert (gap <= G_MARGIN).all(), (np.argwhere(gap > G_MARGIN)[:5], gap.max())
    # log q of the sampled token, where the token agrees
    same = tok == ref.tokens
    assert np.max(np.abs(lq[same] - ref.logq[same])) < 2e-4
    log(f"  tokens bit-exact on {int(ok.sum())}/{rows} confident rows")


def run_verify(drafts, dl, tl, T, seed, rnd, anchor=False, logq=None):
    b, m = drafts.shape
    V = dl.shape[-1]
    acc = torch.full((b,), -1, dtype=torch.int32, device="cuda")
    out = torch.full((b,), -1, dtype=torch.int32, device="cuda")
    anc = torch.full((b,), -1, dtype=torch.int32, device="cuda") if anchor else None
    ws = B.sampling_workspace(b, m + 1, V)
    lq = None if logq is None else torch.from_numpy(logq.astype(np.float32)).cuda()
    B.verify_sampled(torch.from_numpy(drafts.astype(np.int32)).cuda(), torch.from_numpy(dl).cuda(),
                     torch.from_numpy(tl).cuda(), T, seed, rnd, acc, out, ws, anc, draft_logq=lq)
    torch.cuda.synchronize()
    res = (acc.cpu().numpy(), out.cpu().numpy())
    if anchor:
        assert np.array_equal(anc.cpu().numpy(), res[1])
    return res


@pytest.mark.parametrize("with_logq", [False, True])
@pytest.mark.parametrize("b,Bk,V,T,mode", [
    (16, 16, 151936, 1.0, "near"),   # residual pass in 8192-logit splits
    (4, 16, 151936, 1.0, "far"),     # 2048-logit splits (few sequences)
    (1, 16, 151936, 0.9, "far"),     # 1024-logit splits
    (24, 16, 1000, 0.8, "near"),
    (12, 8, 500, 1.2, "far"),
    (6, 16, 300, 1.0, "equal"),
])
def test_gpu_verify_sampled_matches_oracle(b, Bk, V, T, mode, with_logq):
    log(f"case: verify_sampled batch {b} block {Bk} vocab {V} T {T} ({mode}), "
        f"draft log q {'given' if with_logq else 'not given'}")
    m = Bk - 1
    dl = logits((b, m, V), 31, f"vd{V}{mode}", 2.0)
    if mode == "near":    # target close to the draft: long accepted prefixes
        tl = np.concatenate([dl + logits((b, m, V), 32, f"vn{V}", 0.35),
                             logits((b, 1, V), 33, f"vb{V}", 2.0)], axis=1).astype(np.float32)
    elif mode == "far":   # independent target: early rejections, residual draws
        tl = logits((b, Bk, V), 34, f"vf{V}", 2.0)
    else:                 # p == q: every candidate is accepted, bonus from row B-1
        tl = np.concatenate([dl, logits((b, 1, V), 35, f"ve{V}", 2.0)], axis=1)
    drawn = S.sample_drafts(dl.reshape(b * m, V), T, seed=77, rnd=2)
    drafts = drawn.tokens.reshape(b, m)
    ref = S.verify(drafts, dl, tl, T, seed=78, rnd=2)
    # log q of the drawn candidates, as the drafting call returns it (here the
    # oracle's, rounded to fp32)
    acc, out = run_verify(drafts, dl, tl, T, 78, 2, anchor=True,
                          logq=drawn.logq.reshape(b, m) if with_logq else None)
    assert ((acc >= 0) & (acc <= m)).all() and ((out >= 0) & (out < V)).all()
    if mode == "equal":
        assert (acc == m).all() and (ref.accept_len == m).all()
    conf_acc = np.array([np.all(ref.u_margin[s][np.isfinite(ref.u_margin[s])] > U_MARGIN)
                         for s in range(b)])
    assert (acc[conf_acc] == ref.accept_len[conf_acc]).all(), \
        (acc[conf_acc], ref.accept_len[conf_acc])
    conf_out = conf_acc & (ref.g_margin > G_MARGIN)
    assert (out[conf_out] == ref.out_token[conf_out]).all(), \
        np.argwhere((out != ref.out_token) & conf_out)[:5]
    assert conf_out.sum() >= (b + 1) // 2
    # every sequence, near-ties included. A differing accept length flips at
    # the first position where the two disagree, which must be a near-tie of
    # u against alpha; with equal accept lengths the emitted token is within
    # G_MARGIN of the oracle's best perturbed score of that row.
    for s_ in range(b):
        if acc[s_] != ref.accept_len[s_]:
            j = int(min(acc[s_], ref.accept_len[s_]))
            assert j < m and ref.u_margin[s_, j] <= U_MARGIN, (s_, acc[s_], ref.accept_len[s_])
        else:
            gap = ref.scores[s_].max() - ref.scores[s_, out[s_]]
            assert gap <= G_MARGIN, (s_, out[s_], ref.out_token[s_], gap)
    log(f"  accept lengths bit-exact on {int(conf_acc.sum())}/{b}, emitted tokens on "
        f"{int(conf_out.sum())}/{b}; mean accept {acc.mean():.2f}")
