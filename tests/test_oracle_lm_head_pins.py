"""Pins of the LM-head backward oracle to things other than itself: explicit
loops over the defining sums, torch autograd of the forward layer, and
finite differences of a scalar loss through the layer."""

import itertools

import numpy as np
import torch

import oracle


def _case(seed, R=3, V=5, H=4):
    rng = np.random.default_rng(seed)
    return rng.normal(0, 1, (R, V)), rng.normal(0, 1, (V, H)), rng.normal(0, 1, (R, H))


def test_matches_the_defining_sums():
    dz, w, hid = _case(0)
    d_hid, d_w = oracle.lm_head_backward(dz, w, hid)
    R, V = dz.shape
    H = w.shape[1]
    for r, h in itertools.product(range(R), range(H)):
        assert abs(d_hid[r, h] - sum(dz[r, v] * w[v, h] for v in range(V))) < 1e-12
    for v, h in itertools.product(range(V), range(H)):
        assert abs(d_w[v, h] - sum(dz[r, v] * hid[r, h] for r in range(R))) < 1e-12


def test_matches_autograd_of_the_layer():
    dz, w, hid = _case(1, R=7, V=11, H=6)
    ht = torch.tensor(hid, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    zq = ht @ wt.T                      # the layer: logits of each position
    zq.backward(torch.tensor(dz))
    d_hid, d_w = oracle.lm_head_backward(dz, w, hid)
    np.testing.assert_allclose(d_hid, ht.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(d_w, wt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_matches_finite_differences():
    dz, w, hid = _case(2)
    loss = lambda hh, ww: float(np.sum(dz * (hh @ ww.T)))   # d loss / d zq = dz
    d_hid, d_w = oracle.lm_head_backward(dz, w, hid)
    eps = 1e-6
    for (r, h) in [(0, 0), (2, 3), (1, 2)]:
        hp, hm = hid.copy(), hid.copy()
        hp[r, h] += eps
        hm[r, h] -= eps
        assert abs((loss(hp, w) - loss(hm, w)) / (2 * eps) - d_hid[r, h]) < 1e-7
    for (v, h) in [(0, 0), (4, 3), (2, 1)]:
        wp, wm = w.copy(), w.copy()
        wp[v, h] += eps
        wm[v, h] -= eps
        assert abs((loss(hid, wp) - loss(hid, wm)) / (2 * eps) - d_w[v, h]) < 1e-7
