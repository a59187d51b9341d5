"""Pins of the float64 length-head update oracle to things other than itself:
torch autograd of the same loss, torch's own AdamW, closed forms of the first
step and of a zero gradient, finite differences, and the label's edge cases.
The pages print the learning rate (tests/golden/pages_parameters.json) and no
worked example of the update."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_parameters.json")))
LR = GOLDEN["length_head_lr"]


def _case(seed, B=16, H=32, k=16, spread=1.0):
    rng = np.random.default_rng(seed)
    h = rng.normal(0, spread, (B, H))
    w = rng.normal(0, 1.0 / math.sqrt(H), H)
    bias = float(rng.normal(0, 0.3))
    bk = rng.integers(1, k + 1, B)
    acc = np.array([rng.integers(0, b + 1) for b in bk])
    return h, w, bias, acc, bk, k


def _torch_loss(h, w, bias, acc, bk, k):
    ht = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    bt = torch.tensor(bias, dtype=torch.float64, requires_grad=True)
    lab = torch.tensor(acc, dtype=torch.float64) / torch.tensor(np.clip(bk, 1, k), dtype=torch.float64)
    rate = torch.sigmoid(ht @ wt + bt)
    loss = torch.nn.functional.mse_loss(rate, lab)
    loss.backward()
    return loss.item(), rate.detach().numpy(), wt.grad.numpy(), bt.grad.item(), ht.grad.numpy()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_loss_and_gradients_match_torch_autograd(seed):
    h, w, bias, acc, bk, k = _case(seed)
    r = oracle.head_loss_and_grads(h, w, bias, acc, bk, k)
    loss, rate, gw, gb, gh = _torch_loss(h, w, bias, acc, bk, k)
    assert math.isclose(r["loss"], loss, rel_tol=1e-12)
    np.testing.assert_allclose(r["rate"], rate, rtol=1e-12)
    np.testing.assert_allclose(r["g_w"], gw, rtol=1e-10, atol=1e-16)
    assert math.isclose(r["g_bias"], gb, rel_tol=1e-10, abs_tol=1e-16)
    np.testing.assert_allclose(r["g_h"], gh, rtol=1e-10, atol=1e-16)


def test_adamw_steps_match_torch_optimizer():
    h, w, bias, acc, bk, k = _case(3)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    bt = torch.tensor([bias], dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([wt, bt], lr=LR)   # the library's own defaults
    ow, ob, state = w.copy(), bias, None
    for step in range(4):
        hs, _, _, accs, bks, _ = _case(10 + step)
        lab = torch.tensor(accs / np.clip(bks, 1, k), dtype=torch.float64)
        opt.zero_grad()
        loss = torch.nn.functional.mse_loss(torch.sigmoid(torch.tensor(hs) @ wt + bt), lab)
        loss.backward()
        opt.step()
        r = oracle.length_head_update(hs, ow, ob, accs, bks, k, state, lr=LR)
        ow, ob, state = r["w"], r["bias"], r["state"]
        np.testing.assert_allclose(ow, wt.detach().numpy(), rtol=1e-12, atol=1e-15)
        assert math.isclose(ob, bt.item(), rel_tol=1e-12, abs_tol=1e-15)
        st = opt.state[wt]
        np.testing.assert_allclose(state["m_w"], st["exp_avg"].numpy(), rtol=1e-10, atol=1e-20)
        np.testing.assert_allclose(state["v_w"], st["exp_avg_sq"].numpy(), rtol=1e-10, atol=1e-24)
        assert state["t"] == step + 1


def test_first_step_closed_form():
    # t = 1: the bias-corrected moments are g and g^2, so without weight decay
    # each parameter moves by lr * g / (|g| + eps)
    h, w, bias, acc, bk, k = _case(4)
    r = oracle.length_head_update(h, w, bias, acc, bk, k, lr=LR, weight_decay=0.0)
    g = r["g_w"]
    np.testing.assert_allclose(r["w"], w - LR * g / (np.abs(g) + 1e-8), rtol=1e-13, atol=1e-18)
    gb = r["g_bias"]
    assert math.isclose(r["bias"], bias - LR * gb / (abs(gb) + 1e-8), rel_tol=1e-13, abs_tol=1e-18)


def test_exact_prediction_gives_zero_gradient_and_pure_decay():
    # h = 0 and bias = 0 give z = 0, rate 1/2, and acc / b_k = 4 / 8 = 1/2:
    # zero loss and gradients, so AdamW only decays the weights
    B, H, k = 8, 16, 16
    h = np.zeros((B, H))
    w = np.full(H, 0.3)
    acc, bk = np.full(B, 4), np.full(B, 8)
    r = oracle.length_head_update(h, w, 0.0, acc, bk, k, lr=LR)
    assert r["loss"] == 0.0 and np.all(r["g_w"] == 0.0) and r["g_bias"] == 0.0
    np.testing.assert_allclose(r["w"], w * (1.0 - LR * 0.01), rtol=1e-15)
    assert r["bias"] == 0.0


def test_gradient_matches_finite_differences():
    h, w, bias, acc, bk, k = _case(6, B=5, H=6)
    r = oracle.head_loss_and_grads(h, w, bias, acc, bk, k)
    eps = 1e-6
    for j in range(len(w)):
        wp, wm = w.copy(), w.copy()
        wp[j] += eps
        wm[j] -= eps
        fd = (oracle.head_loss_and_grads(h, wp, bias, acc, bk, k)["loss"]
              - oracle.head_loss_and_grads(h, wm, bias, acc, bk, k)["loss"]) / (2 * eps)
        assert abs(fd - r["g_w"][j]) <= 1e-8
    fd = (oracle.head_loss_and_grads(h, w, bias + eps, acc, bk, k)["loss"]
          - oracle.head_loss_and_grads(h, w, bias - eps, acc, bk, k)["loss"]) / (2 * eps)
    assert abs(fd - r["g_bias"]) <= 1e-8
    hp, hm = h.copy(), h.copy()
    hp[2, 3] += eps
    hm[2, 3] -= eps
    fd = (oracle.head_loss_and_grads(hp, w, bias, acc, bk, k)["loss"]
          - oracle.head_loss_and_grads(hm, w, bias, acc, bk, k)["loss"]) / (2 * eps)
    assert abs(fd - r["g_h"][2, 3]) <= 1e-8


def test_label_edges():
    k = 16
    h = np.zeros((5, 4))
    w = np.zeros(4)
    acc = np.array([16, 0, 3, 5, 7])
    bk = np.array([16, 9, 0, -2, 40])   # b_k clamps to [1, k]: 16, 9, 1, 1, 16
    r = oracle.head_loss_and_grads(h, w, 0.0, acc, bk, k)
    np.testing.assert_array_equal(r["label"], [1.0, 0.0, 3.0, 5.0, 7.0 / 16.0])
