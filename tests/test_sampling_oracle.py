"""Pins of the temperature > 0 oracle (oracle/sampling.py), none of which
re-runs its formulas:

  * Philox4x32-10 against the generator's published known-answer vectors
    (tests/golden/philox4x32_10_kat.txt);
  * the Gumbel-max categorical sampler against the softmax law (Monte Carlo);
  * the verification rule against the target law, eq. 8 of the technical
    review ("DFlash: Why a Diffusion Drafter Can Accelerate an Autoregressive
    Model", sec. 4.2), and its acceptance mass 1 - Z, eq. 7 (Monte Carlo);
  * the review's worked example (acceptance totals 0.7, every rejection is
    corrected to token A), as a constructed instance with those properties;
  * the temperature -> 0 limit, which must reduce to the greedy accept rule;
  * planted mistakes (mutations) that one of the pins must catch.
"""
from pathlib import Path

import numpy as np
import pytest

from oracle import dflash_oracle as O
from oracle import sampling as S


GOLDEN = Path(__file__).parent / "golden" / "philox4x32_10_kat.txt"


def kat_vectors():
    out = []
    for line in GOLDEN.read_text().splitlines():
        if line.strip() and not line.startswith("#"):
            w = [int(x, 16) for x in line.split()]
            out.append((w[:4], w[4:6], w[6:]))
    return out


def test_philox_known_answer_vectors():
    vecs = kat_vectors()
    assert len(vecs) == 3
    for counter, key, want in vecs:
        got = S.philox4x32(*[np.uint64(x) for x in counter], np.uint64(key[0]), np.uint64(key[1]))
        assert [int(x) for x in got] == want


def test_philox_known_answer_vectors_as_one_array_call():
    vecs = kat_vectors()
    c = np.array([v[0] for v in vecs], dtype=np.uint64)
    k = np.array([v[1] for v in vecs], dtype=np.uint64)
    got = S.philox4x32(c[:, 0], c[:, 1], c[:, 2], c[:, 3], k[:, 0], k[:, 1])
    for j, (_, _, want) in enumerate(vecs):
        assert [int(got[w][j]) for w in range(4)] == want


def test_philox_refuses_words_of_more_than_32_bits():
    with pytest.raises(AssertionError):
        S.philox4x32(np.uint64(1 << 32), 0, 0, 0, 0, 0)


def test_seed_halves_are_the_key():
    # the 64-bit seed is the key (low word, high word): a seed that differs
    # only in its high half draws different numbers
    a = S.uniforms(5, np.arange(8), 0, 0, 0)
    b = S.uniforms(5 + (1 << 32), np.arange(8), 0, 0, 0)
    assert not np.array_equal(a, b)
    vecs = kat_vectors()
    counter, key, want = vecs[2]
    seed = key[0] | (key[1] << 32)
    u = S.uniforms(seed, np.arange(4) + 4 * counter[0], counter[1], counter[2], counter[3])
    assert np.array_equal(u, (np.array(want, dtype=np.float64) // 512 + 0.5) / (1 << 23))


def test_uniforms_lattice():
    u = S.uniforms(3, np.arange(10000), 5, 2, 0)
    assert np.all(u > 0) and np.all(u < 1)
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)
    assert np.all(((u * (1 << 23)) - 0.5) % 1 == 0)  # on the 23-bit lattice, exact in fp32
    assert abs(u.mean() - 0.5) < 0.01 and abs(u.var() - 1 / 12) < 0.005


def test_row_uniforms_equal_elementwise_definition():
    V = 37
    rows = np.array([0, 3, (1 << 32) - 1])
    a = S.row_uniforms(9, V, rows, 5, 2)
    b = S.uniforms(9, np.arange(V)[None, :], rows[:, None], 5, 2)
    assert np.array_equal(a, b)


def chi2_ok(counts, probs, n):
    exp = probs * n
    keep = exp > 5
    chi2 = float(np.sum((counts[keep] - exp[keep]) ** 2 / exp[keep]))
    dof = int(keep.sum()) - 1
    return chi2 < dof + 6 * np.sqrt(2 * dof) + 10, chi2


def test_gumbel_max_samples_the_softmax_law():
    logits = np.array([1.0, 0.2, -0.5, 2.0, 0.0])
    T = 0.7
    n = 120000
    rows = np.broadcast_to(logits, (n, logits.size))
    d = S.sample_drafts(rows, T, seed=11, rnd=3)
    counts = np.bincount(d.tokens, minlength=logits.size)
    probs = np.exp(logits / T) / np.exp(logits / T).sum()
    ok, chi2 = chi2_ok(counts, probs, n)
    assert ok, (counts / n, probs, chi2)
    assert np.allclose(d.logq, np.log(probs)[d.tokens])


def run_one_position(p, q, n, seed=5):
    """Draw y ~ q and verify one candidate (m = 1) n times; returns the token
    the round emits at that position (y if accepted, else the correction) and
    whether it was accepted."""
    T = 1.0
    V = len(p)
    dl = np.log(q)[None, :].repeat(n, 0)
    d = S.sample_drafts(dl, T, seed=seed, rnd=0)
    tl = np.stack([np.log(p), np.log(p)])[None].repeat(n, 0)
    ver = S.verify(d.tokens[:, None], dl[:, None, :], tl, T, seed=seed + 1, rnd=0)
    emitted = np.where(ver.accept_len == 1, d.tokens, ver.out_token)
    return emitted, ver.accept_len == 1


def test_eq8_output_law_is_the_target_law():
    p = np.array([0.1, 0.45, 0.05, 0.4])
    q = np.array([0.4, 0.1, 0.3, 0.2])
    n = 40000
    emitted, accepted = run_one_position(p, q, n)
    ok, chi2 = chi2_ok(np.bincount(emitted, minlength=4), p, n)
    assert ok, (np.bincount(emitted, minlength=4) / n, chi2)
    # eq. 7: the acceptance probability is sum_z min(p, q) = 1 - Z
    acc = np.minimum(p, q).sum()
    assert abs(accepted.mean() - acc) < 5 * np.sqrt(acc * (1 - acc) / n)


def test_worked_example_acceptance_and_correction():
    # A constructed instance with the review's stated outcome: acceptance
    # totals 0.7 and all of the missing 0.3 mass belongs to token A (index 0),
    # so every rejection is corrected to A.
    p = np.array([0.5, 0.3, 0.2])
    q = np.array([0.2, 0.5, 0.3])
    n = 30000
    emitted, accepted = run_one_position(p, q, n, seed=9)
    assert abs(accepted.mean() - 0.7) < 5 * np.sqrt(0.21 / n)
    assert np.all(emitted[~accepted] == 0)
    ok, _ = chi2_ok(np.bincount(emitted, minlength=3), p, n)
    assert ok


def test_zero_temperature_limit_is_the_greedy_rule():
    rng = np.random.default_rng(3)
    b, m, V = 40, 5, 50
    dl = rng.normal(size=(b, m, V)) * 3
    tl = rng.normal(size=(b, m + 1, V)) * 3
    # make half of the candidate positions agree with the target's argmax
    tl[:, :m] += (rng.random((b, m, 1)) < 0.6) * 50 * np.eye(V)[np.argmax(dl, -1)]
    T = 1e-4
    d = S.sample_drafts(dl.reshape(b * m, V), T, seed=1, rnd=0)
    drafts = d.tokens.reshape(b, m)
    assert np.array_equal(drafts, np.argmax(dl, -1))
    ver = S.verify(drafts, dl, tl, T, seed=2, rnd=0)
    acc_g, bonus_g = O.accept(drafts, np.argmax(tl, -1))
    assert np.array_equal(ver.accept_len, acc_g)
    assert np.array_equal(ver.out_token, bonus_g)


# ---- mutations: each planted mistake must be caught by a pin above ----------

def mutated(monkeypatch, name):
    orig_verify = S.verify

    if name == "alpha_q_over_p":
        # accept with min(1, q/p): swap the roles inside verify
        def bad(drafts, dl, tl, T, seed, rnd):
            return orig_verify(drafts, tl[:, :-1], np.concatenate([dl, tl[:, -1:]], 1), T, seed, rnd)
        monkeypatch.setattr(S, "verify", bad)
    elif name == "residual_from_target":
        def bad(drafts, dl, tl, T, seed, rnd):
            # resampling from the unmodified target on rejection
            v = orig_verify(drafts, dl, tl, T, seed, rnd)
            for s in range(len(v.out_token)):
                a = v.accept_len[s]
                if a < drafts.shape[1]:
                    lp = S.log_softmax(tl[s, a], T)
                    g = S.gumbel(S.uniforms(seed, np.arange(lp.size), s * (drafts.shape[1] + 1) + a, rnd, 2))
                    v.out_token[s] = S.gumbel_argmax(lp, g)[0]
            return v
        monkeypatch.setattr(S, "verify", bad)
    elif name == "gumbel_sign":
        monkeypatch.setattr(S, "gumbel", lambda u: np.log(-np.log(u)))
    elif name == "philox_key_not_bumped":
        monkeypatch.setattr(S, "_W0", np.uint64(0))
        monkeypatch.setattr(S, "_W1", np.uint64(0))
    elif name == "philox_multipliers_swapped":
        m0, m1 = S._M0, S._M1
        monkeypatch.setattr(S, "_M0", m1)
        monkeypatch.setattr(S, "_M1", m0)
    elif name == "temperature_ignored":
        orig_ls = S.log_softmax
        monkeypatch.setattr(S, "log_softmax", lambda logits, T: orig_ls(logits, 1.0))


@pytest.mark.parametrize("name,pin", [
    ("alpha_q_over_p", test_eq8_output_law_is_the_target_law),
    ("residual_from_target", test_worked_example_acceptance_and_correction),
    ("gumbel_sign", test_gumbel_max_samples_the_softmax_law),
    ("temperature_ignored", test_gumbel_max_samples_the_softmax_law),
    ("philox_key_not_bumped", test_philox_known_answer_vectors),
    ("philox_multipliers_swapped", test_philox_known_answer_vectors),
])
def test_mutation_is_caught(monkeypatch, name, pin):
    mutated(monkeypatch, name)
    with pytest.raises(AssertionError):
        pin()
