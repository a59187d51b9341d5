"""Pins of the sampling-verification oracle to things other than itself: the
generator's published known-answer vectors, the uniformity of its output,
the distribution of the exponential race, the published correctness theorem
of speculative sampling (every emitted token is distributed as the target),
the acceptance probability min(1, p/q), and the block semantics."""

import json
import math
import os

import numpy as np
import pytest
import scipy.stats

import oracle

KAT = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")))


@pytest.mark.parametrize("vec", KAT["vectors"])
def test_philox_known_answers(vec):
    c = [int(x, 16) for x in vec["counter"]]
    k = [int(x, 16) for x in vec["key"]]
    out = oracle.philox4x32_10([c[0]], [c[1]], [c[2]], [c[3]], k[0], k[1])
    assert [int(o[0]) for o in out] == [int(x, 16) for x in vec["out"]]


def test_race_uniforms_are_uniform_and_open():
    u = np.concatenate([oracle.race_uniforms(r, 4096, 0x1234_5678_9ABC) for r in range(25)])
    assert 0.0 < u.min() and u.max() < 1.0
    counts, _ = np.histogram(u, bins=64, range=(0.0, 1.0))
    assert scipy.stats.chisquare(counts).pvalue > 1e-4
    # neighbouring words of one counter are not correlated
    assert abs(np.corrcoef(u[:-1], u[1:])[0, 1]) < 0.02


def _logits(p):
    return np.log(np.asarray(p, dtype=np.float64))


def test_exponentials_match_the_series_at_the_extremes():
    # -ln(u) = sum_n (1-u)^n / n, summed exactly in rationals, for words whose
    # u lies within 2^-32 of 1, around 1/2, and at the bottom of the range
    import fractions
    words = [2 ** 32 - 1, 2 ** 32 - 2, 2 ** 32 - 1000, 2 ** 31, 2 ** 31 - 1, 3 * 2 ** 30, 12345, 0]
    got = oracle.exponential_from_word(np.array(words))
    for w, e in zip(words, got):
        u = fractions.Fraction(2 * w + 1, 2 ** 33)
        if 1 - u <= fractions.Fraction(1, 2):
            ref = float(sum((1 - u) ** n / n for n in range(1, 80)))
        else:
            ref = -math.log(float(u))   # u <= 1/2: the library log is exact to an ulp here
        assert math.isclose(e, ref, rel_tol=1e-14), (w, e, ref)


def test_exponential_race_draws_the_residual_distribution():
    # p - q has residual mass on entries 0, 2, 3 (normalised: 0.2, 0.5, 0.3)
    p = np.array([0.3, 0.1, 0.5, 0.1])
    q = np.array([0.1, 0.4, 0.0 + 1e-300, 0.4 - 1e-300])
    q = q / q.sum()
    r = np.maximum(0, p - q)
    want = r / r.sum()
    n = 20000
    draws = np.array([int(np.argmax(oracle.residual_keys(_logits(p), _logits(q), row, 7)[1]))
                      for row in range(n)])
    counts = np.bincount(draws, minlength=4)
    assert counts[1] == 0
    keep = want > 0
    assert scipy.stats.chisquare(counts[keep], want[keep] * n).pvalue > 1e-4


def test_acceptance_probability_is_min_one_p_over_q():
    rng = np.random.default_rng(1)
    p = np.array([0.2, 0.5, 0.3])
    q = np.array([0.5, 0.25, 0.25])
    for d, want in ((0, 0.4), (1, 1.0), (2, 1.0)):
        u = rng.random(20000)
        acc = np.array([oracle.accept_test(_logits(p), _logits(q), d, x)[0] for x in u])
        assert abs(acc.mean() - want) < 4 * math.sqrt(want * (1 - want) / len(u)) + 1e-12


def test_emitted_token_is_distributed_as_the_target():
    # The published theorem: drafting from q, accepting with min(1, p/q) and
    # drawing rejections from the residual emits tokens distributed as p.
    rng = np.random.default_rng(2)
    V = 6
    p = rng.dirichlet(np.ones(V))
    q = rng.dirichlet(np.ones(V))
    zp, zq = _logits(p), _logits(q)
    n = 20000
    emitted = np.empty(n, dtype=np.int64)
    for t in range(n):
        d = int(rng.choice(V, p=q))
        # a fresh seed per trial gives every trial its own residual race
        res = oracle.spec_verify(zp[None, :], zq[None, :], [d], np.array([rng.random()]), k=1,
                                 seed=1000 + t, bk=np.array([1]))
        emitted[t] = d if res["acc"][0] == 1 else res["token"][0]
    counts = np.bincount(emitted, minlength=V)
    assert scipy.stats.chisquare(counts, p * n).pvalue > 1e-4


def test_block_semantics():
    rng = np.random.default_rng(3)
    V, k = 50, 4
    zp = rng.normal(0, 1, (2 * k, V))
    zq = zp.copy()
    zq[1] += rng.normal(0, 3, V)              # position 1 of request 0 differs from the target
    draft = np.argmax(zq, axis=1)
    u = np.full(2 * k, 0.999)
    # request 0: p = q at position 0 (always accepted); position 1 is rejected
    # when q(d) > p(d) / 0.999; request 1: p = q everywhere
    pd = np.exp(zp[1, draft[1]] - np.log(np.exp(zp[1]).sum()))
    qd = np.exp(zq[1, draft[1]] - np.log(np.exp(zq[1]).sum()))
    assert 0.999 * qd > pd
    res = oracle.spec_verify(zp, zq, draft, u, k=k, seed=5, bk=np.array([4, 3]))
    assert list(res["acc"]) == [1, 3]
    assert res["token"][1] == -1 and res["rejected_row"][1] == -1
    r1 = np.maximum(0, np.exp(zp[1] - np.log(np.exp(zp[1]).sum())) - np.exp(zq[1] - np.log(np.exp(zq[1]).sum())))
    assert r1[res["token"][0]] > 0                 # the draw has residual mass
    # out-of-range drafts are rejected; b_k clamps to [1, k]
    d2 = draft.copy()
    d2[0], d2[4] = -1, V
    res = oracle.spec_verify(zp, zq, d2, u, k=k, seed=5, bk=np.array([0, 9]))
    assert list(res["acc"]) == [0, 0]
    # a forced rejection where p = q draws from p itself
    res = oracle.spec_verify(zp, zq, draft, u, k=k, seed=5, bk=np.array([4, 4]), force={4: False})
    assert res["acc"][1] == 0 and 0 <= res["token"][1] < V


def test_race_keys_follow_their_definition_on_a_tiny_row():
    # brute force: the key of entry j is max(0, p_j - q_j) / -ln(u_j) with u_j
    # from word j % 4 of the generator at counter (j // 4, row, 0, 0)
    zp = np.array([0.5, -1.0, 2.0, 0.0, 1.5])
    zq = np.array([0.0, 0.5, 1.0, 0.2, -2.0])
    seed, row = (0xDEADBEEF << 32) | 0x12345, 77
    r, key, p, q = oracle.residual_keys(zp, zq, row, seed)
    for j in range(5):
        words = oracle.philox4x32_10([j // 4], [row], [0], [0], seed & 0xFFFFFFFF, seed >> 32)
        u = (int(words[j % 4][0]) + 0.5) / 2 ** 32
        assert math.isclose(oracle.race_exponentials(row, 5, seed)[j], -math.log(u), rel_tol=1e-9)
        pj = math.exp(zp[j]) / sum(math.exp(x) for x in zp)
        qj = math.exp(zq[j]) / sum(math.exp(x) for x in zq)
        assert math.isclose(key[j], max(0.0, pj - qj) / -math.log(u), rel_tol=1e-12, abs_tol=0)
