"""Pins of the float64 oracle to things other than itself.

Each test checks the oracle against a closed form, a library routine, an
invariant of the mathematics, brute force, finite differences, or the pages'
own Eq. (1) (Pith review page, Referee Report minor comment 1, paper Sec. 2.1).
The pages print no worked example of the loss, gradient or length head; the
printed hyperparameters live in tests/golden/pages_parameters.json.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_parameters.json")))
ALPHA = GOLDEN["mixing_alpha"]
DELTA = GOLDEN["clip_delta"]
GAMMA = GOLDEN["length_scale_gamma"]


def _rows(seed, V, scale=2.0, noise=1.0):
    rng = np.random.default_rng(seed)
    zp = rng.normal(0, scale, V)
    zq = zp + rng.normal(0, noise, V)
    return zp, zq


# ---------------------------------------------------------------------------
# number decoding
# ---------------------------------------------------------------------------

def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, 100000, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    bits = bits[exp != 0xFF]  # finite encodings only
    ours = oracle.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------------------
# length head
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("k", [16, 32, 15])
def test_length_head_zero_preactivation_gives_half(k):
    h = np.zeros((1, 8), np.float32)
    w = np.ones(8, np.float32)
    rate, bk_c, _ = oracle.length_head(h, w, 0.0, 1.0, k, "ceil")
    _, bk_f, _ = oracle.length_head(h, w, 0.0, 1.0, k, "floor")
    assert rate[0] == 0.5
    assert bk_c[0] == math.ceil(k / 2) and bk_f[0] == k // 2


def test_length_head_saturation_and_clamp():
    w = np.ones(4, np.float32)
    hi = np.full((1, 4), 20.0, np.float32)
    lo = np.full((1, 4), -20.0, np.float32)
    for mode in ("ceil", "floor"):
        assert oracle.length_head(hi, w, 0.0, 1.0, 16, mode)[1][0] == 16
        assert oracle.length_head(lo, w, 0.0, 1.0, 16, mode)[1][0] == 1
    # gamma above 1 would overshoot k; the clamp keeps b_k <= k
    assert oracle.length_head(np.zeros((1, 4), np.float32), w, 0.0, 3.0, 16)[1][0] == 16


def test_length_head_matches_scipy_expit_and_ceil_characterisation():
    rng = np.random.default_rng(3)
    H, B, k = 256, 64, 16
    w = rng.normal(0, 1, H).astype(np.float32)
    h = rng.normal(0, 0.2, (B, H)).astype(np.float32)
    bias = 0.25
    rate, bk, margin = oracle.length_head(h, w, bias, GAMMA, k)
    ref = scipy.special.expit(h.astype(np.float64) @ w.astype(np.float64) + bias)
    np.testing.assert_allclose(rate, ref, rtol=1e-13, atol=0)
    for b in range(B):
        x = GAMMA * ref[b] * k
        if margin[b] < 1e-9:
            continue
        n = int(bk[b])
        # ceil(x) is the unique integer n with n - 1 < x <= n (then clamped)
        assert (n - 1 < x <= n) or (n == 1 and x <= 1) or (n == k and x > k)
    _, bkf, _ = oracle.length_head(h, w, bias, 0.5, k, "floor")
    for b in range(B):
        x = 0.5 * ref[b] * k
        n = int(bkf[b])
        assert (n <= x < n + 1) or (n == 1 and x < 1)


# ---------------------------------------------------------------------------
# target argmax and acceptance
# ---------------------------------------------------------------------------

def test_argmax_ties_lowest_index_bruteforce():
    rng = np.random.default_rng(5)
    for _ in range(200):
        V = int(rng.integers(1, 40))
        row = rng.integers(-3, 4, V).astype(np.float64)  # many exact ties
        best = max(row)
        first = [j for j in range(V) if row[j] == best][0]
        assert oracle.target_argmax(row) == first
    assert oracle.target_argmax(np.array([-0.0, 0.0, -1.0])) == 0  # -0 == +0


def test_accepted_length_exhaustive():
    k = 6
    for pattern in itertools.product([True, False], repeat=k):
        tgt = list(range(k))
        draft = [t if m else t + 100 for t, m in zip(tgt, pattern)]
        for b in range(0, k + 1):
            head = list(pattern[:b])
            expect = head.index(False) if False in head else b
            assert oracle.accepted_length(draft, tgt, b) == expect


@pytest.mark.parametrize("acc_rate,k,b", [(0.8, 16, 16), (0.5, 16, 16), (0.9, 32, 32), (0.7, 16, 5)])
def test_accepted_length_matches_eq1_closed_form(acc_rate, k, b):
    """Eq. (1): with i.i.d. acceptance the expected tokens per step
    (accepted draft tokens + bonus) is (1 - Acc^(k+1)) / (1 - Acc); truncated
    at b positions the accepted-draft part is sum_{i=1..b} Acc^i."""
    rng = np.random.default_rng(11)
    n = 40000
    match = rng.random((n, k)) < acc_rate
    draft = np.where(match, 0, 1)
    tgt = np.zeros(k, dtype=np.int64)
    accs = np.array([oracle.accepted_length(draft[t], tgt, b) for t in range(n)], dtype=np.float64)
    if b == k:
        expect = (1 - acc_rate ** (k + 1)) / (1 - acc_rate) - 1.0
    else:
        expect = sum(acc_rate ** i for i in range(1, b + 1))
    sigma = accs.std() / math.sqrt(n)
    assert abs(accs.mean() - expect) < 4 * sigma + 1e-12


# ---------------------------------------------------------------------------
# OPD loss: library routines and closed forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(4))
def test_ce_branch_matches_torch_cross_entropy(seed):
    zp, zq = _rows(seed, 500)
    t = oracle.row_terms(zp, zq, lam=1.0, tau=DELTA)
    a = int(np.argmax(zp))
    ref = torch.nn.functional.cross_entropy(torch.tensor(zq)[None], torch.tensor([a])).item()
    assert abs(t.loss - ref) <= 1e-12 * abs(ref)
    assert abs(t.ce - ref) <= 1e-12 * abs(ref)


@pytest.mark.parametrize("seed", range(4))
def test_unclipped_reverse_kl_matches_scipy_rel_entr(seed):
    zp, zq = _rows(seed, 700, noise=1.5)
    t = oracle.row_terms(zp, zq, lam=0.0, tau=1e9)
    p = scipy.special.softmax(zp)
    q = scipy.special.softmax(zq)
    ref = float(np.sum(scipy.special.rel_entr(q, p)))  # KL(q || p): reverse KL
    assert ref > 0
    assert abs(t.loss - ref) <= 1e-10 * ref
    # and it is not the forward KL
    fwd = float(np.sum(scipy.special.rel_entr(p, q)))
    assert abs(t.loss - fwd) > 1e-3 * ref


def test_kl_zero_when_drafter_equals_target():
    zp, _ = _rows(7, 300)
    for shift in (0.0, 3.25):
        t = oracle.row_terms(zp, zp + shift, lam=0.0, tau=0.1)
        assert abs(t.klc) < 1e-12 and abs(t.loss) < 1e-12
        assert np.max(np.abs(t.grad)) < 1e-15
        t2 = oracle.row_terms(zp, zp + shift, lam=0.5, tau=0.1)
        lp = scipy.special.log_softmax(zp)
        a = int(np.argmax(zp))
        assert abs(t2.loss - 0.5 * (-lp[a])) < 1e-12


@pytest.mark.parametrize("V", [2, 64, 4096])
def test_ce_is_log_v_on_uniform_drafter(V):
    zp, _ = _rows(9, V)
    t = oracle.row_terms(zp, np.zeros(V), lam=1.0, tau=0.1)
    assert abs(t.ce - math.log(V)) < 1e-12
    t0 = oracle.row_terms(np.zeros(V), np.zeros(V), lam=0.5, tau=0.1)
    assert abs(t0.loss - 0.5 * math.log(V)) < 1e-12


def test_negative_branch_worked_example():
    """Two-token vocabulary, p = (0.9, 0.1), q = (0.3, 0.7).
    r_0 = 0.3 ln(1/3) ~ -0.330 (negative branch), r_1 = 0.7 ln 7 ~ 1.362."""
    zp = np.log([0.9, 0.1])
    zq = np.log([0.3, 0.7])
    r0 = 0.3 * math.log(0.3 / 0.9)
    r1 = 0.7 * math.log(0.7 / 0.1)
    # tau = 0.5: r_0 inside, r_1 clipped to +0.5
    t = oracle.row_terms(zp, zq, lam=0.5, tau=0.5)
    assert t.argmax == 0
    assert list(t.c) == [True, False]
    assert abs(t.klc - (r0 + 0.5)) < 1e-15
    S = 0.3 * (math.log(1 / 3) + 1)
    assert abs(t.S - S) < 1e-15
    ce = -math.log(0.3)
    assert abs(t.loss - (0.5 * ce + 0.5 * (r0 + 0.5))) < 1e-15
    g0 = 0.5 * (0.3 - 1.0) + 0.5 * 0.3 * ((math.log(1 / 3) + 1) - S)
    g1 = 0.5 * 0.7 + 0.5 * 0.7 * (0.0 - S)
    np.testing.assert_allclose(t.grad, [g0, g1], rtol=0, atol=1e-15)
    # tau = 0.1: both clipped, opposite signs; no KL gradient at all
    t = oracle.row_terms(zp, zq, lam=0.0, tau=0.1)
    assert list(t.c) == [False, False]
    assert abs(t.klc - (-0.1 + 0.1)) < 1e-15
    assert np.max(np.abs(t.grad)) == 0.0
    # tau = 2: nothing clipped, KL = r0 + r1
    t = oracle.row_terms(zp, zq, lam=0.0, tau=2.0)
    assert abs(t.klc - (r0 + r1)) < 1e-15


def test_clip_bound_and_small_tau_limit():
    zp, zq = _rows(13, 2000, noise=3.0)
    for tau in (0.1, DELTA, 1e-3):
        t = oracle.row_terms(zp, zq, lam=0.0, tau=tau)
        clipped = np.clip(t.r, -tau, tau)
        assert np.all(np.abs(clipped) <= tau)
        assert abs(t.klc) <= np.count_nonzero(t.r) * tau
    t = oracle.row_terms(zp, zq, lam=0.0, tau=1e-14)
    assert abs(t.klc) <= 2000 * 1e-14


# ---------------------------------------------------------------------------
# gradient: finite differences, autograd, invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("lam,tau", [(0.0, 0.05), (0.5, 0.1), (ALPHA, DELTA), (1.0, 0.1), (0.3, 1e9)])
@pytest.mark.parametrize("seed", range(3))
def test_gradient_central_finite_differences(lam, tau, seed):
    V = 48
    zp, zq = _rows(100 + seed, V, noise=2.5)
    t = oracle.row_terms(zp, zq, lam, tau)
    h = 1e-6
    for j in range(V):
        up = zq.copy()
        up[j] += h
        dn = zq.copy()
        dn[j] -= h
        tu = oracle.row_terms(zp, up, lam, tau)
        td = oracle.row_terms(zp, dn, lam, tau)
        if not (np.array_equal(tu.c, t.c) and np.array_equal(td.c, t.c)):
            continue  # a clip kink sits inside the stencil
        fd = (tu.loss - td.loss) / (2 * h)
        assert abs(fd - t.grad[j]) <= 2e-7 + 1e-6 * abs(t.grad[j]), (j, fd, t.grad[j])


@pytest.mark.parametrize("lam,tau", [(0.5, 0.1), (0.0, 0.05), (ALPHA, DELTA), (0.2, 1e9)])
def test_gradient_matches_torch_autograd(lam, tau):
    zp, zq = _rows(21, 3000, noise=3.0)
    t = oracle.row_terms(zp, zq, lam, tau, grad_scale=0.25)
    zp_t = torch.tensor(zp)
    zq_t = torch.tensor(zq, requires_grad=True)
    logq = torch.log_softmax(zq_t, 0)
    logp = torch.log_softmax(zp_t, 0)
    a = int(torch.argmax(zp_t))
    kl_terms = logq.exp() * (logq - logp)
    loss = lam * (-logq[a]) + (1 - lam) * torch.clamp(kl_terms, -tau, tau).sum()
    (0.25 * loss).backward()
    assert abs(loss.item() - t.loss) <= 1e-12 * max(1.0, abs(t.loss))
    np.testing.assert_allclose(t.grad, zq_t.grad.numpy(), rtol=1e-9, atol=1e-16)


@pytest.mark.parametrize("lam,tau", [(0.5, 0.1), (0.0, 1e9), (1.0, 0.05)])
def test_shift_invariance_and_zero_row_sum(lam, tau):
    zp, zq = _rows(31, 1000, noise=2.0)
    t = oracle.row_terms(zp, zq, lam, tau)
    s = oracle.row_terms(zp - 7.5, zq + 11.0, lam, tau)
    assert s.argmax == t.argmax
    assert abs(s.loss - t.loss) < 1e-11
    np.testing.assert_allclose(s.grad, t.grad, rtol=0, atol=1e-13)
    assert abs(t.grad.sum()) < 1e-13


# ---------------------------------------------------------------------------
# the batch pass: masks, layouts, reductions
# ---------------------------------------------------------------------------

def _batch(seed, B, k, V):
    rng = np.random.default_rng(seed)
    zp = rng.normal(0, 2, (B * k, V))
    zq = zp + rng.normal(0, 0.7, (B * k, V))
    draft = np.argmax(zq, axis=1)
    return zp, zq, draft


def test_dense_mask_and_reductions():
    B, k, V = 5, 6, 40
    zp, zq, draft = _batch(41, B, k, V)
    bk = np.array([0, 1, 3, 6, 99])  # 0 and 99 are clamped to 1 and k
    out = oracle.verify_opd(zp, zq, draft, k=k, lam=0.5, tau=0.1, grad_scale=2.0, bk=bk)
    eff = np.clip(bk, 1, k)
    for b in range(B):
        for i in range(k):
            r = b * k + i
            assert out["tgt_argmax"][r] == int(np.argmax(zp[r]))
            if i < eff[b]:
                t = oracle.row_terms(zp[r], zq[r], 0.5, 0.1, 2.0)
                assert out["row_loss"][r] == t.loss
                assert np.array_equal(out["grad"][r], t.grad)
            else:
                assert out["row_loss"][r] == 0.0 and not out["grad"][r].any()
                assert not out["row_stats"][r].any()
        assert 0 <= out["acc_len"][b] <= eff[b]
        assert abs(out["req_loss"][b] - sum(out["row_loss"][b * k:(b + 1) * k])) < 1e-12
    assert abs(out["total_loss"] - out["req_loss"].sum()) < 1e-12


def test_ragged_layout_agrees_with_dense_on_verified_rows():
    B, k, V = 6, 5, 33
    zp, zq, draft = _batch(43, B, k, V)
    draft[::3] = np.argmax(zp[::3], axis=1)  # make some positions accept
    bk = np.array([1, 5, 2, 3, 4, 1])
    dense = oracle.verify_opd(zp, zq, draft, k=k, lam=0.3, tau=0.05, bk=bk)
    keep = np.concatenate([np.arange(b * k, b * k + bk[b]) for b in range(B)])
    row_off = np.concatenate([[0], np.cumsum(bk)])
    rag = oracle.verify_opd(zp[keep], zq[keep], draft[keep], k=k, lam=0.3, tau=0.05, row_off=row_off)
    assert np.array_equal(rag["acc_len"], dense["acc_len"])
    np.testing.assert_array_equal(rag["row_loss"], dense["row_loss"][keep])
    np.testing.assert_array_equal(rag["grad"], dense["grad"][keep])
    np.testing.assert_allclose(rag["req_loss"], dense["req_loss"], rtol=0, atol=1e-14)


def test_out_of_range_draft_never_matches():
    B, k, V = 2, 4, 20
    zp, zq, _ = _batch(47, B, k, V)
    tgt = np.argmax(zp, axis=1)
    draft = tgt.copy()
    draft[1] = -1
    draft[k + 2] = V
    out = oracle.verify_opd(zp, zq, draft, k=k, lam=0.5, tau=0.1, bk=np.array([4, 4]))
    assert list(out["acc_len"]) == [1, 2]


def test_clip_interval_is_closed():
    """Reading: an entry exactly on the threshold counts as inside the clip
    interval (the convention of torch.clamp's gradient).  Set tau to one
    entry's |r_j| exactly and check that entry still passes gradient."""
    zp, zq = _rows(17, 200, noise=3.0)
    t = oracle.row_terms(zp, zq, lam=0.0, tau=1e9)
    j = int(np.argmax(np.abs(t.r)))
    tau = float(abs(t.r[j]))
    t2 = oracle.row_terms(zp, zq, lam=0.0, tau=tau)
    assert t2.c[j]
    # torch.clamp passes gradient on the boundary too
    x = torch.tensor([tau, -tau, tau * 1.5], dtype=torch.float64, requires_grad=True)
    torch.clamp(x, -tau, tau).sum().backward()
    assert list(x.grad.numpy()) == [1.0, 1.0, 0.0]


# ---------------------------------------------------------------------------
# the helpers that decide which GPU decisions must match bit for bit
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("k,gamma,x,want", [
    (16, 1.0, 4.8, 0.2), (16, 1.0, 8.5, 0.5), (16, 1.0, 3.25, 0.25), (16, 1.0, 15.9, 0.1),
    (16, 1.0, 0.3, 0.3), (32, 1.0, 20.75, 0.25), (16, 0.5, 5.6, 0.4), (16, 1.0, 12.0, 0.0),
    (16, 1.0, 8.0, 0.0), (32, 1.0, 7.0, 0.0),
])
def test_length_head_margin_hand_computed(k, gamma, x, want):
    """margin is the distance of gamma * rate * k to the nearest integer.
    With one input of width 1, w = 1 and bias 0, the pre-activation z is the
    input itself; z = log(s / (1 - s)) for s = x / (gamma k) makes
    gamma * sigmoid(z) * k = x up to float64 rounding (about 1e-15)."""
    s = x / (gamma * k)
    z = math.log(s / (1.0 - s))
    h = np.array([[z]], np.float64)
    w = np.array([1.0], np.float64)
    for mode in ("ceil", "floor"):
        rate, bk, margin = oracle.length_head(h, w, 0.0, gamma, k, mode)
        assert abs(rate[0] - s) < 1e-14
        assert abs(margin[0] - want) < 1e-12
        if want > 1e-9:  # away from an integer the rounding is unambiguous
            n = math.ceil(x) if mode == "ceil" else math.floor(x)
            assert bk[0] == min(max(n, 1), k)
        else:            # on an integer the oracle flags the decision
            assert margin[0] <= 1e-9


def test_clip_margin_hand_computed():
    """clip_margin is ||r_j| - tau| / tau: 0 on either edge of the interval,
    growing with the distance from it, the same for r and -r."""
    r = np.array([0.1, -0.1, 0.05, -0.2, 0.1001, 0.0, -0.0999, 0.3])
    want = np.array([0.0, 0.0, 0.5, 1.0, 0.001, 1.0, 0.001, 2.0])
    np.testing.assert_allclose(oracle.clip_margin(r, 0.1), want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.clip_margin(r * 7.0, 0.7), want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", ["tiny", "single", "concurrent", "long"])
def test_seeded_workloads_have_no_ambiguous_verification_lengths(name):
    """Every b_k of the seeded workloads, under each (gamma, bias) pair the GPU
    tests use, lies more than 1e-9 from a rounding boundary, so the GPU tests
    can require every b_k bit for bit."""
    import synth
    w = synth.make(name, V=64)
    for gamma, bias in [(w.gamma, w.bias), (1.0, 0.0), (0.75, 0.3), (1.6, -2.0)]:
        for mode in ("ceil", "floor"):
            _, _, margin = oracle.length_head(w.h, w.w, bias, gamma, w.k, mode)
            assert margin.min() > 1e-9, (name, gamma, bias, mode, margin.min())
