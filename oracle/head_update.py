"""Plain float64 oracle for the online update of the adaptive length head.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path may import it.

Sources (the pages, cited by title and section):
  [P1] Pith verdict record for arXiv 2607.19223 (JSON): skeptic critique,
       "load-bearing attack" (the head is trained on the verification
       outcome of the truncated block).
  [P3] Pith review page "AdaFlash: Adaptive Speculative Decoding via
       On-Policy Distilled Diffusion Drafters": Referee Report major
       comment 1 (paper Sec. 3.2, "Online Update of the Length Head": an MSE
       loss against the observed acceptance rate a*) and minor comment 2
       (the head outputs one scalar); "Axiom & Free-Parameter Ledger"
       (length head learning rate 2e-4, optimiser AdamW).

What is computed, per request b of one verification step:
  rate_b  = sigmoid(w . h_b + bias)                 the head's prediction  [P3 minor 2]
  label_b = acc_b / b_k,b                           observed acceptance    [P3 major 1]
  loss    = mean_b (rate_b - label_b)^2             MSE                    [P3 major 1]
then the gradients of loss with respect to w, bias and h, and one AdamW step
on (w, bias) with learning rate 2e-4                                       [P3 ledger]

Readings where the pages leave a step open (each is listed in the design
notes with its reason):
  * the label's denominator is b_k, the verified length: the acceptance
    status of positions at or beyond b_k is never observed (the referee's
    point), so acc / b_k is the only label the step can form.  b_k is
    clamped to [1, k] as in the verification pass.
  * the MSE is the mean over the B requests of the step.
  * AdamW's other constants are not printed; the defaults of the common
    implementation are used (beta1 0.9, beta2 0.999, eps 1e-8, decoupled
    weight decay 0.01), with bias correction and the step count t counted
    from 1.
"""

from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

ADAMW_DEFAULTS = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _sigmoid(z: float) -> float:
    if z >= 0.0:
        return 1.0 / (1.0 + math.exp(-z))
    e = math.exp(z)
    return e / (1.0 + e)


def head_loss_and_grads(h: np.ndarray, w: np.ndarray, bias: float, acc: np.ndarray, bk: np.ndarray,
                        k: int) -> Dict[str, np.ndarray]:
    """MSE of the predicted acceptance rate against acc / b_k and its
    gradients.  h [B, H], w [H]; acc, bk [B] integers.

    With e_b = rate_b - label_b and s_b = rate_b (1 - rate_b) (the sigmoid's
    derivative), d loss / d z_b = 2 e_b s_b / B, and by the chain rule
    g_w = sum_b dz_b h_b, g_bias = sum_b dz_b, g_h[b] = dz_b w.
    """
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, H = h.shape
    rate = np.empty(B)
    label = np.empty(B)
    dz = np.empty(B)
    sq = np.empty(B)
    for b in range(B):
        z = math.fsum((w * h[b]).tolist()) + float(bias)
        rate[b] = _sigmoid(z)
        n = min(max(int(bk[b]), 1), k)
        label[b] = int(acc[b]) / n
        e = rate[b] - label[b]
        sq[b] = e * e
        dz[b] = 2.0 * e * rate[b] * (1.0 - rate[b]) / B
    g_w = np.array([math.fsum((dz * h[:, j]).tolist()) for j in range(H)])
    g_bias = math.fsum(dz.tolist())
    g_h = dz[:, None] * w[None, :]
    loss = math.fsum(sq.tolist()) / B
    return dict(rate=rate, label=label, loss=loss, dz=dz, g_w=g_w, g_bias=g_bias, g_h=g_h)


def adamw_step(theta: np.ndarray, g: np.ndarray, m: np.ndarray, v: np.ndarray, t: int, *,
               lr: float, beta1: float, beta2: float, eps: float, weight_decay: float):
    """One AdamW step (decoupled weight decay, bias-corrected moments) on a
    parameter array; t is the number of this step, counted from 1.
    Returns the new (theta, m, v)."""
    theta = np.asarray(theta, dtype=np.float64) * (1.0 - lr * weight_decay)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    bc1 = 1.0 - beta1 ** t
    bc2 = 1.0 - beta2 ** t
    theta = theta - (lr / bc1) * m / (np.sqrt(v) / math.sqrt(bc2) + eps)
    return theta, m, v


def length_head_update(h: np.ndarray, w: np.ndarray, bias: float, acc: np.ndarray, bk: np.ndarray,
                       k: int, state: Optional[dict] = None, **hyper) -> dict:
    """One online update of the length head from one verification step.

    state holds the optimiser moments and the step count:
    m_w, v_w [H], m_b, v_b (scalars), t (steps taken so far; 0 for a fresh
    head).  Returns the loss, predictions, labels and gradients, the updated
    w and bias, and the new state (t advanced by one)."""
    p = dict(ADAMW_DEFAULTS)
    p.update(hyper)
    H = np.asarray(w).shape[0]
    if state is None:
        state = dict(m_w=np.zeros(H), v_w=np.zeros(H), m_b=0.0, v_b=0.0, t=0)
    r = head_loss_and_grads(h, w, bias, acc, bk, k)
    t = int(state["t"]) + 1
    w_new, m_w, v_w = adamw_step(w, r["g_w"], state["m_w"], state["v_w"], t, **p)
    b_arr, m_b, v_b = adamw_step(np.array([float(bias)]), np.array([r["g_bias"]]),
                                 np.array([float(state["m_b"])]), np.array([float(state["v_b"])]), t, **p)
    r.update(w=w_new, bias=float(b_arr[0]),
             state=dict(m_w=m_w, v_w=v_w, m_b=float(m_b[0]), v_b=float(v_b[0]), t=t))
    return r
