"""Plain float64 oracle for the backward of the drafter's LM head.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path may import it.

Source: the Pith review page "AdaFlash: Adaptive Speculative Decoding via
On-Policy Distilled Diffusion Drafters" ("Axiom & Free-Parameter Ledger":
drafter learning rate, AdamW updates of the drafter): the OPD gradient with
respect to the drafter logits is propagated into the drafter, whose last
layer maps the hidden state of each position to its logits,
zq[r, v] = sum_h hid[r, h] W[v, h].  The step after the verify + OPD pass
is therefore that layer's backward:
  d hid[r, h] = sum_v dz[r, v] W[v, h]       (dz @ W)
  d W[v, h]   = sum_r dz[r, v] hid[r, h]     (dz^T @ hid)
Reading: the layer has no bias, and its inputs are the bfloat16 values the
caller stores (decoded exactly); the sums are exact float64 sums.
"""

from __future__ import annotations

import numpy as np


def lm_head_backward(dz: np.ndarray, w: np.ndarray, hid: np.ndarray):
    """dz [R, V], w [V, H], hid [R, H] (float64 values) -> (d_hid [R, H],
    d_w [V, H]), the two products written as the definitions above."""
    dz = np.asarray(dz, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    hid = np.asarray(hid, dtype=np.float64)
    return dz @ w, dz.T @ hid
