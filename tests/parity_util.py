"""Helpers shared by the GPU parity tests: move seeded workloads to the GPU,
run the HIP path through the binding, and compare with the float64 oracle.

Acceptance rule (the arithmetic behind it is written out in the design notes):
  * bit-exact: target argmax, accepted lengths, b_k (except b_k decisions the
    oracle flags as within 1e-9 of an integer);
  * row loss, clipped-KL sum, S: |gpu - ref| <= 1e-3 |ref| + 1e-5;
  * lse_p, lse_q: |gpu - ref| <= 2e-6 |ref| + 2e-6;
  * gradient, per entry: |gpu - ref| <= 1e-3 |ref| + 2e-5 gs q_j (1 + |ell_j| + |S|)
    -- the second term bounds float32 rounding of q_j, ell_j and S where the
    reference itself cancels to near zero; with a reverse-KL temperature
    T != 1 that term is scaled by 1 / T (the KL part's factor) and
    2e-5 gs q1_j is added for the cross-entropy part's own softmax q1;
    an entry other than the label whose q_j (and q1_j) lies below the
    smallest normal float32, 2^-126 (a logit about 87 below the row's
    log-sum-exp), may read anything between 0 and the reference: the float32
    exponential flushes such q_j to zero;
  * lse of zq at temperature 1 (lse_q1): as lse_p, lse_q;
  * an entry whose |r_j| lies within w_j of tau may be classified either way
    by float32, where w_j bounds |r32_j - r_j| from the GPU's own log-sum-exp
    errors (measured on the row) and float32 rounding of the entry's steps
    (clip_window); rows with such entries are accepted if they match the
    oracle with any combination of those indicators flipped (at most 3).
    AMBIGUOUS counts the entries and rows this rule touched.
"""

from __future__ import annotations

import itertools
import math
from typing import Iterable, Optional

import numpy as np
import torch

import oracle
import synth

LOSS_RTOL, LOSS_ATOL = 1e-3, 1e-5
LSE_RTOL, LSE_ATOL = 2e-6, 2e-6
GRAD_RTOL, GRAD_QTOL = 1e-3, 2e-5
FLT_MIN_NORMAL = 2.0 ** -126  # smallest normal float32
U32 = 2.0 ** -24  # unit roundoff of float32
AMBIGUOUS = {"rows": 0, "entries": 0}


def clip_window(t: oracle.RowTerms, zp_row, zq_row, tau: float, d_lse_p: float, d_lse_q: float) -> np.ndarray:
    """Width of the band around tau in which the GPU's float32 r_j may fall on
    the other side of tau than the float64 r_j.

    The GPU forms q_j = exp2(fma(s zq_j, L, -lse_q L)) and
    ell_j = s (zq_j - zp_j) - (lse_q - lse_p) (s = 1 / T, L = log2 e / T in
    float32) from its float32 log-sum-exps, then r_j = q_j ell_j.  To first
    order, with dq, dp the log-sum-exp errors:
      q32 / q - 1   within  eq = dq + 4 u (1 + |s zq_j| + |lse_q|)
                            (the exponent's roundings; exp2 to 1 ulp)
      ell32 - ell   within  el = dq + dp + 4 u (1 + |s (zq_j - zp_j)| + |lse_q - lse_p|)
      r32 - r       within  q (|ell| (eq + u) + el)
    plus |tau32 - tau| <= u tau for the threshold itself; the band is twice
    that bound."""
    s = 1.0 / t.temperature
    eq = d_lse_q + 4 * U32 * (1.0 + np.abs(s * zq_row) + abs(t.lse_q))
    el = d_lse_q + d_lse_p + 4 * U32 * (1.0 + np.abs(s * (zq_row - zp_row)) + abs(t.lse_q - t.lse_p))
    return 2.0 * (t.q * (np.abs(t.ell) * (eq + U32) + el) + U32 * tau)


def logits_tensor(a: np.ndarray, dtype: str, dev="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def decode_rows(w: synth.Workload, which: str, rows) -> np.ndarray:
    a = (w.zp if which == "zp" else w.zq)[rows]
    if w.dtype == "bf16":
        return oracle.bf16_bits_to_f64(a)
    return a.astype(np.float64)


def gpu_inputs(w: synth.Workload, dev="cuda") -> dict:
    d = dict(zp=logits_tensor(w.zp, w.dtype, dev), zq=logits_tensor(w.zq, w.dtype, dev),
             draft=torch.from_numpy(w.draft.astype(np.int32)).to(dev))
    if w.row_off is not None:
        d["row_off"] = torch.from_numpy(w.row_off.astype(np.int32)).to(dev)
    return d


def run_fwd(av, inp: dict, w: synth.Workload, *, bk: Optional[np.ndarray], lam: float, tau: float,
            gs: float = 1.0, vecs: int = 0, want_grad: bool = True, temperature: float = 1.0,
            split: int = 0) -> dict:
    kw = dict(k=w.k, lam=lam, tau=tau, grad_scale=gs, onchip_limit=vecs, want_grad=want_grad,
              temperature=temperature, split_rows=split)
    if w.row_off is not None:
        kw["row_off"] = inp["row_off"]
    else:
        kw["bk"] = torch.from_numpy(np.asarray(bk, dtype=np.int32)).to(inp["zp"].device)
    out = av.av_verify_opd_fwd(inp["zp"], inp["zq"], inp["draft"], **kw)
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in out.items()}


def spans(w: synth.Workload, bk: Optional[np.ndarray]):
    """(first row, stored rows, effective b_k) per request."""
    if w.row_off is not None:
        n = np.diff(w.row_off)
        return [(int(w.row_off[b]), int(n[b]), int(n[b])) for b in range(w.B)]
    return [(b * w.k, w.k, min(max(int(bk[b]), 1), w.k)) for b in range(w.B)]


def close(a, b, rtol, atol) -> bool:
    return abs(float(a) - float(b)) <= rtol * abs(float(b)) + atol


def grad_row_ok(g: np.ndarray, t: oracle.RowTerms, gs: float) -> np.ndarray:
    scale = t.q * (1.0 + np.abs(t.ell) + abs(t.S))
    if t.temperature != 1.0:
        scale = scale / t.temperature + t.q1
    tol = GRAD_RTOL * np.abs(t.grad) + GRAD_QTOL * abs(gs) * scale
    flushed = t.q < FLT_MIN_NORMAL
    if t.q1 is not None:
        flushed &= t.q1 < FLT_MIN_NORMAL
    flushed[t.argmax] = False
    g64 = g.astype(np.float64)
    between = (np.abs(g64) <= np.abs(t.grad)) & (g64 * t.grad >= 0.0)
    return (np.abs(g64 - t.grad) <= tol) | (flushed & between)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (8 significant bits; below the
    smallest normal, the subnormal spacing 2^-133)."""
    m, e = np.frexp(np.abs(x))
    return np.where(np.abs(x) >= 2.0 ** -126, np.ldexp(1.0, e - 8), 2.0 ** -133)


def grad_row_ok_bf16(g: np.ndarray, t: oracle.RowTerms, gs: float) -> np.ndarray:
    """A bfloat16 gradient entry is the float32 entry rounded to nearest: it
    may differ from the float64 reference by the float32 bar plus one
    bfloat16 spacing (half of one for the rounding, half as margin)."""
    scale = t.q * (1.0 + np.abs(t.ell) + abs(t.S))
    if t.temperature != 1.0:
        scale = scale / t.temperature + t.q1
    g64 = g.astype(np.float64)
    tol = GRAD_RTOL * np.abs(t.grad) + GRAD_QTOL * abs(gs) * scale
    tol = tol + bf16_ulp(np.maximum(np.abs(t.grad), np.abs(g64)) + tol)
    flushed = t.q < FLT_MIN_NORMAL
    if t.q1 is not None:
        flushed &= t.q1 < FLT_MIN_NORMAL
    flushed[t.argmax] = False
    between = (np.abs(g64) <= np.abs(t.grad)) & (g64 * t.grad >= 0.0)
    return (np.abs(g64 - t.grad) <= tol) | (flushed & between)


def check_row(r: int, out: dict, zp_row, zq_row, lam, tau, gs, verified: bool, errors: list,
              temperature: float = 1.0):
    """Compare one row of GPU output with the oracle; append messages to errors."""
    a_ref = oracle.target_argmax(zp_row)
    if int(out["tgt_argmax"][r]) != a_ref:
        errors.append(f"row {r}: argmax {out['tgt_argmax'][r]} != {a_ref}")
    grad = out.get("grad")
    stats = out.get("row_stats")
    lse1 = out.get("lse_q1")
    if not verified:
        if lse1 is not None and lse1[r] != 0.0:
            errors.append(f"row {r}: unverified row has lse_q1 {lse1[r]}")
        if out["row_loss"][r] != 0.0:
            errors.append(f"row {r}: unverified loss {out['row_loss'][r]}")
        if grad is not None and np.any(grad[r] != 0.0):
            errors.append(f"row {r}: unverified row has a nonzero gradient")
        if stats is not None and np.any(stats[r] != 0.0):
            errors.append(f"row {r}: unverified row has nonzero stats")
        return
    t = oracle.row_terms(zp_row, zq_row, lam, tau, gs, temperature=temperature)
    variants = [t]
    amb = []
    if math.isfinite(tau):
        if stats is not None:  # the GPU's own log-sum-exp errors on this row
            d_p, d_q = abs(float(stats[r][0]) - t.lse_p), abs(float(stats[r][1]) - t.lse_q)
        else:                  # the bound the lse check allows
            d_p = LSE_RTOL * abs(t.lse_p) + LSE_ATOL
            d_q = LSE_RTOL * abs(t.lse_q) + LSE_ATOL
        w = clip_window(t, zp_row, zq_row, tau, d_p, d_q)
        amb = np.nonzero(np.abs(np.abs(t.r) - tau) <= w)[0]
        if len(amb):
            AMBIGUOUS["rows"] += 1
            AMBIGUOUS["entries"] += len(amb)
    if 0 < len(amb) <= 3:
        for flips in itertools.product([False, True], repeat=len(amb)):
            if any(flips):
                ov = {int(j): (not bool(t.c[j])) if f else bool(t.c[j]) for j, f in zip(amb, flips)}
                variants.append(oracle.row_terms(zp_row, zq_row, lam, tau, gs, clip_override=ov,
                                                 temperature=temperature))
    msgs = None
    for v in variants:
        m = []
        if not close(out["row_loss"][r], v.loss, LOSS_RTOL, LOSS_ATOL):
            m.append(f"loss {out['row_loss'][r]} vs {v.loss}")
        if stats is not None:
            s = stats[r]
            if not close(s[0], v.lse_p, LSE_RTOL, LSE_ATOL):
                m.append(f"lse_p {s[0]} vs {v.lse_p}")
            if not close(s[1], v.lse_q, LSE_RTOL, LSE_ATOL):
                m.append(f"lse_q {s[1]} vs {v.lse_q}")
            if not close(s[2], v.S, LOSS_RTOL, LOSS_ATOL):
                m.append(f"S {s[2]} vs {v.S}")
            if not close(s[3], v.klc, LOSS_RTOL, LOSS_ATOL):
                m.append(f"KLc {s[3]} vs {v.klc}")
        if lse1 is not None and not close(lse1[r], v.lse_q1, LSE_RTOL, LSE_ATOL):
            m.append(f"lse_q1 {lse1[r]} vs {v.lse_q1}")
        if grad is not None:
            ok = grad_row_ok(grad[r], v, gs)
            if not ok.all():
                j = int(np.argmin(ok))
                m.append(f"grad: {np.count_nonzero(~ok)} entries off, e.g. j={j} {grad[r][j]} vs {v.grad[j]}")
        if not m:
            return
        if msgs is None:
            msgs = m
    errors.append(f"row {r}: " + "; ".join(msgs))


# State the forked workers of check_workload read (set before the pool starts).
_POOL: dict = {}


def _check_chunk(rows):
    """Worker: check_row over a list of rows; returns (errors, ambiguous counts)."""
    c = _POOL
    AMBIGUOUS["rows"] = AMBIGUOUS["entries"] = 0
    errors: list = []
    for r in rows:
        check_row(r, c["out"], decode_rows(c["w"], "zp", r), decode_rows(c["w"], "zq", r), c["lam"], c["tau"],
                  c["gs"], bool(c["verified"][r]), errors, temperature=c["temperature"])
        if len(errors) >= c["max_errors"]:
            break
    return errors, dict(AMBIGUOUS)


def _check_rows(out, w, verified, rows, lam, tau, gs, temperature, max_errors, workers):
    """check_row over `rows`: in this process, or in `workers` forked
    processes that read the workload and the GPU outputs from this process's
    memory (they run only the float64 oracle; nothing there touches the GPU)."""
    rows = list(rows)
    if workers <= 1 or len(rows) < 2 * workers:
        errors: list = []
        for r in rows:
            check_row(r, out, decode_rows(w, "zp", r), decode_rows(w, "zq", r), lam, tau, gs,
                      bool(verified[r]), errors, temperature=temperature)
            if len(errors) >= max_errors:
                break
        return errors
    import multiprocessing as mp
    _POOL.update(out=out, w=w, verified=verified, lam=lam, tau=tau, gs=gs, temperature=temperature,
                 max_errors=max_errors)
    chunks = [rows[i::4 * workers] for i in range(4 * workers)]
    errors = []
    try:
        with mp.get_context("fork").Pool(workers) as pool:
            for e, amb in pool.imap_unordered(_check_chunk, chunks):
                errors.extend(e)
                AMBIGUOUS["rows"] += amb["rows"]
                AMBIGUOUS["entries"] += amb["entries"]
    finally:
        _POOL.clear()
    return errors[:max_errors]


def check_workload(out: dict, w: synth.Workload, bk: Optional[np.ndarray], lam: float, tau: float,
                   gs: float = 1.0, rows: Optional[Iterable[int]] = None, max_errors: int = 10,
                   temperature: float = 1.0, workers: int = 0):
    """Full comparison (rows=None) or comparison on sampled rows; argmax and
    acceptance are always checked on every row and request.  workers > 1 runs
    the per-row comparisons in that many forked processes."""
    errors: list = []
    sp = spans(w, bk)
    verified = np.zeros(w.R, dtype=bool)
    for r0, n, bkb in sp:
        verified[r0:r0 + bkb] = True
    # argmax of every row and acceptance of every request: exact
    tgt_ref = np.empty(w.R, dtype=np.int64)
    for r in range(w.R):
        tgt_ref[r] = oracle.target_argmax(decode_rows(w, "zp", r))
    bad = np.nonzero(out["tgt_argmax"] != tgt_ref)[0]
    if len(bad):
        errors.append(f"argmax differs on {len(bad)} rows, e.g. row {bad[0]}: "
                      f"{out['tgt_argmax'][bad[0]]} vs {tgt_ref[bad[0]]}")
    for b, (r0, n, bkb) in enumerate(sp):
        acc = oracle.accepted_length(w.draft[r0:r0 + n], tgt_ref[r0:r0 + n], bkb)
        if int(out["acc_len"][b]) != acc:
            errors.append(f"request {b}: acc {out['acc_len'][b]} vs {acc}")
    # per-row loss / stats / gradient
    check = range(w.R) if rows is None else rows
    errors.extend(_check_rows(out, w, verified, check, lam, tau, gs, temperature, max_errors, workers))
    # reductions: per request from the (already checked) row losses, in float64
    rl = out["row_loss"].astype(np.float64)
    for b, (r0, n, bkb) in enumerate(sp):
        ref = math.fsum(rl[r0:r0 + bkb].tolist())
        if not close(out["req_loss"][b], ref, 1e-6, 1e-6):
            errors.append(f"request {b}: req_loss {out['req_loss'][b]} vs sum of rows {ref}")
    tot = math.fsum(out["req_loss"].astype(np.float64).tolist())
    if not close(out["total_loss"][0], tot, 1e-6, 1e-5):
        errors.append(f"total {out['total_loss'][0]} vs {tot}")
    if int(out["status"][0]) != 0:
        errors.append(f"device status {out['status'][0]}")
    return errors


def oracle_reductions(w: synth.Workload, bk, lam, tau, gs=1.0, temperature=1.0) -> dict:
    """Whole-batch oracle (small workloads only)."""
    zp = decode_rows(w, "zp", slice(None))
    zq = decode_rows(w, "zq", slice(None))
    if w.row_off is not None:
        return oracle.verify_opd(zp, zq, w.draft, k=w.k, lam=lam, tau=tau, grad_scale=gs,
                                 row_off=w.row_off, want_grad=False, temperature=temperature)
    return oracle.verify_opd(zp, zq, w.draft, k=w.k, lam=lam, tau=tau, grad_scale=gs, bk=bk,
                             want_grad=False, temperature=temperature)
