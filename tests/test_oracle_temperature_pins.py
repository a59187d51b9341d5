"""Pins of the oracle's reverse-KL temperature to things other than itself.

Reading pinned here (the Pith review page of AdaFlash, "Axiom &
Free-Parameter Ledger", names a reverse-KL temperature without defining it):
the reverse-KL term compares softmax(zp / T) with softmax(zq / T), the hard
cross-entropy keeps the plain softmax of zq, and no T^2 factor is applied.

Each check uses a library routine (scipy's KL divergence and log-softmax,
torch autograd), finite differences, or an identity of the mathematics
(scaling the logits by 1 / T at T = 1; the CE term's independence of T).
"""

import math

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle

TEMPS = [0.25, 0.5, 2.0, 7.3]


def _rows(seed, V, scale=2.0, noise=1.0):
    rng = np.random.default_rng(seed)
    zp = rng.normal(0, scale, V)
    zq = zp + rng.normal(0, noise, V)
    return zp, zq


@pytest.mark.parametrize("T", TEMPS)
def test_unclipped_kl_term_is_scipy_kl_of_tempered_softmaxes(T):
    zp, zq = _rows(1, 300)
    t = oracle.row_terms(zp, zq, lam=0.0, tau=1e30, temperature=T)
    p = scipy.special.softmax(zp / T)
    q = scipy.special.softmax(zq / T)
    assert t.loss == pytest.approx(scipy.stats.entropy(q, p), rel=1e-10, abs=1e-14)
    assert t.lse_p == pytest.approx(scipy.special.logsumexp(zp / T), rel=1e-13)
    assert t.lse_q == pytest.approx(scipy.special.logsumexp(zq / T), rel=1e-13)
    assert t.lse_q1 == pytest.approx(scipy.special.logsumexp(zq), rel=1e-13)


@pytest.mark.parametrize("T", TEMPS)
def test_cross_entropy_term_does_not_depend_on_temperature(T):
    zp, zq = _rows(2, 200)
    a = int(np.argmax(zp))
    t = oracle.row_terms(zp, zq, lam=1.0, tau=0.05, grad_scale=1.5, temperature=T)
    ls = scipy.special.log_softmax(zq)
    assert t.loss == pytest.approx(-ls[a], rel=1e-12)
    ref = np.exp(ls)
    ref[a] -= 1.0
    np.testing.assert_allclose(t.grad, 1.5 * ref, rtol=1e-11, atol=1e-15)


@pytest.mark.parametrize("T", TEMPS)
def test_kl_term_equals_unit_temperature_pass_on_scaled_logits(T):
    # lam = 0: the loss at T is the T = 1 loss of (zp / T, zq / T); by the
    # chain rule its gradient in zq is 1 / T times that pass's gradient
    zp, zq = _rows(3, 400, scale=3.0)
    for tau in (1e30, 0.01, 0.002):
        a = oracle.row_terms(zp, zq, lam=0.0, tau=tau, grad_scale=0.7, temperature=T)
        b = oracle.row_terms(zp / T, zq / T, lam=0.0, tau=tau, grad_scale=0.7)
        assert a.loss == pytest.approx(b.loss, rel=1e-12, abs=1e-15)
        assert a.S == pytest.approx(b.S, rel=1e-12, abs=1e-15)
        np.testing.assert_allclose(a.grad, b.grad / T, rtol=1e-11, atol=1e-16)


def _torch_loss(zp, zq, a, lam, tau, T):
    logp = torch.log_softmax(zp / T, 0)
    logq = torch.log_softmax(zq / T, 0)
    kl = torch.clamp(logq.exp() * (logq - logp), -tau, tau).sum()
    ce = -torch.log_softmax(zq, 0)[a]
    return lam * ce + (1.0 - lam) * kl


@pytest.mark.parametrize("T", TEMPS)
@pytest.mark.parametrize("lam,tau", [(0.5, 0.01), (0.2, 0.003), (0.8, 1e9)])
def test_gradient_matches_torch_autograd(T, lam, tau):
    zp, zq = _rows(4, 500, scale=2.5)
    t = oracle.row_terms(zp, zq, lam=lam, tau=tau, grad_scale=2.0, temperature=T)
    assert np.min(oracle.clip_margin(t.r, tau)) > 1e-6  # no entry sits on the clip boundary
    zpt = torch.tensor(zp, dtype=torch.float64)
    zqt = torch.tensor(zq, dtype=torch.float64, requires_grad=True)
    loss = _torch_loss(zpt, zqt, t.argmax, lam, tau, T)
    (g,) = torch.autograd.grad(2.0 * loss, zqt)
    assert t.loss == pytest.approx(loss.item(), rel=1e-12, abs=1e-15)
    np.testing.assert_allclose(t.grad, g.numpy(), rtol=1e-10, atol=1e-15)


@pytest.mark.parametrize("T", [0.5, 3.0])
def test_gradient_matches_central_differences(T):
    zp, zq = _rows(5, 7, scale=1.5)
    lam, tau = 0.4, 0.05
    t = oracle.row_terms(zp, zq, lam=lam, tau=tau, temperature=T)
    assert np.min(oracle.clip_margin(t.r, tau)) > 1e-3
    h = 1e-6
    for m in range(len(zq)):
        up, dn = zq.copy(), zq.copy()
        up[m] += h
        dn[m] -= h
        fd = (oracle.row_terms(zp, up, lam, tau, temperature=T).loss
              - oracle.row_terms(zp, dn, lam, tau, temperature=T).loss) / (2 * h)
        assert t.grad[m] == pytest.approx(fd, rel=1e-6, abs=1e-9)


def test_high_temperature_flattens_the_kl_term():
    # both tempered softmaxes tend to uniform, so KL(q_T || p_T) -> 0 like 1 / T^2
    zp, zq = _rows(6, 100)
    kl = [oracle.row_terms(zp, zq, 0.0, 1e30, temperature=T).loss for T in (1e2, 1e3)]
    assert 0.0 <= kl[1] < kl[0] < 1e-3
    assert kl[0] / kl[1] == pytest.approx(100.0, rel=0.05)


def test_batch_pass_reports_tempered_stats_and_plain_lse():
    rng = np.random.default_rng(7)
    R, V, k = 6, 50, 3
    zp = rng.normal(0, 2, (R, V))
    zq = zp + rng.normal(0, 1, (R, V))
    out = oracle.verify_opd(zp, zq, np.zeros(R, np.int64), k=k, lam=0.3, tau=0.02,
                            bk=np.array([2, 3]), temperature=1.7)
    for r in range(R):
        if not out["verified"][r]:
            assert out["lse_q1"][r] == 0.0 and not out["row_stats"][r].any()
            continue
        assert out["row_stats"][r][0] == pytest.approx(scipy.special.logsumexp(zp[r] / 1.7), rel=1e-13)
        assert out["row_stats"][r][1] == pytest.approx(scipy.special.logsumexp(zq[r] / 1.7), rel=1e-13)
        assert out["lse_q1"][r] == pytest.approx(scipy.special.logsumexp(zq[r]), rel=1e-13)


def test_nonpositive_temperature_is_rejected():
    zp, zq = _rows(8, 10)
    for T in (0.0, -1.0, math.nan):
        with pytest.raises(ValueError):
            oracle.row_terms(zp, zq, 0.5, 0.1, temperature=T)
