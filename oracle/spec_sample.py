"""Plain float64 oracle for sampling-based block verification (speculative
sampling) of a drafted block.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path may import it.

Sources: the Pith review page "AdaFlash: Adaptive Speculative Decoding via
On-Policy Distilled Diffusion Drafters" lists, in its "Axiom &
Free-Parameter Ledger", the standard speculative-decoding acceptance formula
(attributed to Leviathan et al. 2023) as an axiom, and its reference list
cites Chen et al. 2023, "Accelerating large language model decoding with
speculative sampling".  The pages print neither algorithm; this file restates
the published method:
  * position i of a block is accepted with probability min(1, p_i(d_i) / q_i(d_i))
    (p: target, q: drafter distribution at that position), in order, and
    the block stops at the first rejection;
  * at the first rejected position the emitted token is drawn from the
    residual distribution max(0, p - q) / sum(max(0, p - q)).
Together these make every emitted token distributed exactly as the target
would have sampled it (the published correctness theorem, pinned by Monte
Carlo in the tests).

Readings (listed in the design notes with their reasons):
  * the acceptance test for position i of request b uses a uniform u in
    [0, 1) supplied by the caller: accept iff u * q(d) < p(d) (the min(1, .)
    is implicit); a draft token outside [0, V) is rejected;
  * only the verified positions i < b_k are tested (b_k clamped to [1, k]);
  * the residual draw uses the exponential-race form of the Gumbel-max
    method: with independent E_j ~ Exp(1), argmax_j r_j / E_j is distributed
    as r / sum(r).  E_j = -ln(u_j) with u_j from the Philox4x32-10
    counter-based generator (Salmon et al., SC 2011), keyed by a 64-bit seed,
    counter (j // 4, row, 0, 0), output word j % 4, u = (word + 1/2) / 2^32;
  * a residual that is zero everywhere (p = q at the rejected position, which
    a rejection can only meet through rounding) is replaced by p itself;
  * a request whose verified positions are all accepted emits no
    replacement (token -1): the bonus token after the block is drawn by the
    caller from the target's next distribution, as for greedy verification;
  * temperature 1 (plain softmax), as for the OPD pass.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

# Philox4x32-10 constants (Salmon et al. 2011): round multipliers and the
# Weyl increments of the key schedule.
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32 with 10 rounds on arrays of counters (uint32 values held in
    int64/uint64 arrays).  Each round multiplies words 0 and 2 by the round
    constants, takes the high and low halves of the 64-bit products, and
    mixes them with words 1 and 3 and the round key; the key is bumped by the
    Weyl constants between rounds.  Returns the four output words."""
    c0 = np.asarray(c0, dtype=np.uint64) & MASK32
    c1 = np.asarray(c1, dtype=np.uint64) & MASK32
    c2 = np.asarray(c2, dtype=np.uint64) & MASK32
    c3 = np.asarray(c3, dtype=np.uint64) & MASK32
    k0 = np.uint64(k0 & MASK32)
    k1 = np.uint64(k1 & MASK32)
    for rnd in range(10):
        if rnd > 0:
            k0 = np.uint64((int(k0) + PHILOX_W0) & MASK32)
            k1 = np.uint64((int(k1) + PHILOX_W1) & MASK32)
        p0 = c0 * np.uint64(PHILOX_M0)   # < 2^64: exact in uint64
        p1 = c2 * np.uint64(PHILOX_M1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def race_words(row: int, V: int, seed: int) -> np.ndarray:
    """The generator words behind the residual draw at stored row `row`."""
    j = np.arange(V, dtype=np.uint64)
    words = philox4x32_10(j >> np.uint64(2), np.full(V, row, dtype=np.uint64), np.zeros(V), np.zeros(V),
                          seed & MASK32, (seed >> 32) & MASK32)
    sel = (j & np.uint64(3)).astype(np.int64)
    return np.choose(sel, words).astype(np.int64)


def race_uniforms(row: int, V: int, seed: int) -> np.ndarray:
    """The uniforms u_j = (word_j + 1/2) / 2^32, j < V, of the residual draw."""
    return (race_words(row, V, seed).astype(np.float64) + 0.5) / 4294967296.0


def exponential_from_word(w: np.ndarray) -> np.ndarray:
    """E = -ln(u) for u = (w + 1/2) / 2^32.  For u >= 1/2 it is formed as
    -log1p(-(1 - u)) from 1 - u = (2^32 - 1 - w + 1/2) / 2^32, which keeps
    full relative precision where u is close to 1 (the same value, computed
    stably)."""
    w = np.asarray(w, dtype=np.int64)
    u = (w.astype(np.float64) + 0.5) / 4294967296.0
    v = ((4294967295 - w).astype(np.float64) + 0.5) / 4294967296.0
    return np.where(u < 0.5, -np.log(u), -np.log1p(-v))


def race_exponentials(row: int, V: int, seed: int) -> np.ndarray:
    """E_j = -ln(u_j), j < V, of the residual draw at stored row `row`."""
    return exponential_from_word(race_words(row, V, seed))


def residual_keys(zp_row: np.ndarray, zq_row: np.ndarray, row: int, seed: int):
    """Residual r = max(0, p - q) of one row and the race keys r_j / E_j."""
    zp = np.asarray(zp_row, dtype=np.float64)
    zq = np.asarray(zq_row, dtype=np.float64)
    p = np.exp(zp - _logsumexp(zp))
    q = np.exp(zq - _logsumexp(zq))
    r = np.maximum(0.0, p - q)
    if not np.any(r > 0.0):   # p = q: nothing to correct, draw from p
        r = p
    e = race_exponentials(row, len(zp), seed)
    return r, r / e, p, q


def _logsumexp(z: np.ndarray) -> float:
    m = float(np.max(z))
    return m + math.log(math.fsum(np.exp(z - m).tolist()))


def accept_test(zp_row: np.ndarray, zq_row: np.ndarray, d: int, u: float):
    """(accepted, margin) for one position: accepted iff u q(d) < p(d); the
    margin |u q(d) - p(d)| / (p(d) + u q(d)) says how close the decision is."""
    V = len(zp_row)
    if not 0 <= int(d) < V:
        return False, math.inf
    zp = np.asarray(zp_row, dtype=np.float64)
    zq = np.asarray(zq_row, dtype=np.float64)
    pd = math.exp(zp[d] - _logsumexp(zp))
    qd = math.exp(zq[d] - _logsumexp(zq))
    a, b = float(u) * qd, pd
    margin = abs(a - b) / (a + b) if a + b > 0.0 else math.inf
    return a < b, margin


def spec_verify(zp: np.ndarray, zq: np.ndarray, draft: Sequence[int], u: np.ndarray, *, k: int,
                seed: int, bk: Optional[np.ndarray] = None, row_off: Optional[np.ndarray] = None,
                force: Optional[dict] = None) -> dict:
    """Sampling-based verification of B drafted blocks.

    Dense layout (row_off None): row b*k+i is position i of request b,
    verified when i < clamp(bk[b], 1, k).  Ragged: request b owns rows
    row_off[b]..row_off[b+1]-1, all verified.  zp, zq float64 [R, V]; u [R]
    the caller's uniforms.  `force` maps a row to a forced accept decision
    (used by tests when a decision lies within rounding of the boundary).

    Returns acc [B] (accepted positions), token [B] (the residual draw at
    the first rejected position, -1 if none was rejected), and per row the
    accept decisions and margins; for each request with a rejection, the
    rejected row and the race keys of that row.
    """
    zp = np.asarray(zp, dtype=np.float64)
    zq = np.asarray(zq, dtype=np.float64)
    R, V = zp.shape
    if row_off is None:
        B = R // k
        spans = [(b * k, min(max(int(bk[b]), 1), k)) for b in range(B)]
    else:
        B = len(row_off) - 1
        spans = [(int(row_off[b]), int(row_off[b + 1] - row_off[b])) for b in range(B)]
    force = force or {}
    acc = np.zeros(B, dtype=np.int64)
    token = np.full(B, -1, dtype=np.int64)
    accept = np.zeros(R, dtype=bool)
    margin = np.full(R, math.inf)
    rejected_row = np.full(B, -1, dtype=np.int64)
    keys = {}
    for b, (r0, n) in enumerate(spans):
        i = 0
        while i < n:
            r = r0 + i
            a, m = accept_test(zp[r], zq[r], int(draft[r]), float(u[r]))
            if r in force:
                a = bool(force[r])
            accept[r], margin[r] = a, m
            if not a:
                break
            i += 1
        acc[b] = i
        if i < n:
            r = r0 + i
            _, key, _, _ = residual_keys(zp[r], zq[r], r, seed)
            token[b] = int(np.argmax(key))
            rejected_row[b] = r
            keys[b] = key
    return dict(acc=acc, token=token, accept=accept, margin=margin, rejected_row=rejected_row, keys=keys)
