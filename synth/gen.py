"""Seeded synthetic logit blocks for the AdaFlash verify + OPD pass.

The pages evaluate on GSM8K, MathQA, code and chat suites with Qwen3 targets
and a DFlash drafter; none of those are available here, so every input is
synthetic and seeded.  The shapes follow the workloads of the hot path:

  tiny        B=1,   k=16, V=4096,   fp32 logits, length-head width H=256
  single      B=1,   k=16, V=151936, bf16,        H=4096
  concurrent  B=128, k=16, V=151936, bf16,        H=4096 (planted head)
  ragged      B=128, k=16, V=151936, bf16, rows packed by b_k ~ p(b) ~ 1/b
  long        B=64,  k=32, V=262144, bf16,        H=5120

V=151936 is the LM-head width of the Qwen3 targets the pages use.

Recipe (all randomness from numpy PCG64 streams keyed by SeedSequence):
  * request b draws from stream [seed, cfg, 0, b]:
      - (per-request noise configs only) sigma_b ~ U(lo, hi), first draw;
      - target logits zp ~ N(0, 2^2) for all of the request's rows;
      - one planted peak per row: +6 at an index drawn uniformly;
      - drafter logits zq = zp + N(0, sigma_i^2), where sigma_i rises
        linearly over the block positions (endpoints included) or is the
        request's sigma_b;
    the values are formed in float64 and then rounded once to the logit
    dtype (round-to-nearest-even to bf16, or to float32);
  * draft token of a row = first index of the largest rounded drafter logit
    (what a greedy drafter would propose);
  * length-head inputs come from stream [seed, cfg, 1]: w ~ N(0, 1/H) then
    h ~ N(0, 1/H) per request (float64, rounded to float32), bias 0.  For
    the concurrent workload the pooled state is planted so that the head's
    pre-activation equals logit(t_b), t_b = clip((4 - sigma_b)/3.7, 1e-3,
    1 - 1e-3): requests with less drafter noise get longer verification
    blocks and b_k spreads over 1..k instead of clustering at k/2;
  * the ragged workload draws b_k from stream [seed, cfg, 2]: a categorical
    over 1..k with p(b) proportional to 1/b, and stores only those rows.

Nothing here computes a verification result, a loss or a gradient.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "CONFIGS",
    "Workload",
    "make",
    "request_rows",
    "to_bf16_bits",
    "bf16_bits_to_float",
]

# name -> (config id used in seeds, parameters)
CONFIGS: Dict[str, dict] = {
    "tiny": dict(cid=1, B=1, k=16, V=4096, dtype="f32", H=256,
                 sigma=("ramp", 0.5, 3.0), bk="head", layout="dense",
                 lam=0.5, tau=0.1),
    "single": dict(cid=2, B=1, k=16, V=151936, dtype="bf16", H=4096,
                   sigma=("ramp", 0.5, 3.0), bk="head", layout="dense",
                   lam=0.5, tau=0.1),
    "concurrent": dict(cid=3, B=128, k=16, V=151936, dtype="bf16", H=4096,
                       sigma=("uniform", 0.3, 4.0), bk="planted", layout="dense",
                       lam=0.5, tau=0.1),
    "ragged": dict(cid=4, B=128, k=16, V=151936, dtype="bf16", H=4096,
                   sigma=("uniform", 0.3, 4.0), bk="inv_b", layout="ragged",
                   lam=0.5, tau=0.1),
    "long": dict(cid=5, B=64, k=32, V=262144, dtype="bf16", H=5120,
                 sigma=("ramp", 0.5, 5.0), bk="head", layout="dense",
                 lam=0.5, tau=0.1),
}

TARGET_STD = 2.0
PEAK = 6.0


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (round to nearest, ties to even), once.

    Works on the float64 bit pattern: bfloat16 keeps 7 of float64's 52 stored
    mantissa bits, so the low 45 bits are rounded away with the usual
    add-half-minus-one-plus-lsb rule (a carry propagates into the exponent as
    it should).  The result is then exactly representable in float32 and its
    upper 16 bits are the bfloat16 encoding.  Finite inputs in the normal
    float32 range only.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    bits = x.view(np.uint64)
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    bits = (bits + (np.uint64((1 << 44) - 1) + lsb)) & np.uint64(~((1 << 45) - 1) & 0xFFFFFFFFFFFFFFFF)
    f32 = bits.view(np.float64).astype(np.float32)
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """bfloat16 encodings -> float32 values (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# workload container
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    dtype: str            # "bf16" (zp/zq hold uint16 encodings) or "f32"
    B: int
    k: int
    V: int
    H: int
    layout: str           # "dense" (row b*k+i) or "ragged" (rows packed by row_off)
    lam: float
    tau: float
    gamma: float
    round_mode: str       # "ceil" or "floor"
    zp: np.ndarray        # [R, V] target logits
    zq: np.ndarray        # [R, V] drafter logits
    draft: np.ndarray     # [R] int32 draft tokens
    row_off: Optional[np.ndarray]  # [B+1] int32 (ragged) else None
    h: Optional[np.ndarray]        # [B, H] float32 pooled drafter state
    w: Optional[np.ndarray]        # [H] float32 length-head weights
    bias: float

    @property
    def R(self) -> int:
        return int(self.zp.shape[0])

    def rows_of(self, b: int) -> Tuple[int, int]:
        """First row and number of stored rows of request b."""
        if self.layout == "ragged":
            return int(self.row_off[b]), int(self.row_off[b + 1] - self.row_off[b])
        return b * self.k, self.k

    def logits_f64(self, which: str, rows=None) -> np.ndarray:
        a = self.zp if which == "zp" else self.zq
        if rows is not None:
            a = a[rows]
        if self.dtype == "bf16":
            return bf16_bits_to_float(a).astype(np.float64)
        return a.astype(np.float64)


# --------------------------------------------------------------------------
# generation
# --------------------------------------------------------------------------

def _cfg(name: str, overrides: dict) -> dict:
    if name not in CONFIGS:
        raise KeyError(f"unknown workload {name!r}; choose from {sorted(CONFIGS)}")
    c = dict(CONFIGS[name])
    for key, val in overrides.items():
        if key not in c:
            raise KeyError(f"unknown override {key!r}")
        c[key] = val
    return c


def _stream(seed: int, cid: int, *path: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cid, *path])))


def _request_sigma(c: dict, rng: np.random.Generator, n_rows: int) -> np.ndarray:
    mode, lo, hi = c["sigma"]
    if mode == "uniform":
        s = rng.uniform(lo, hi)
        return np.full(n_rows, s)
    k = c["k"]
    pos = np.arange(n_rows, dtype=np.float64)
    return lo + (hi - lo) * pos / max(k - 1, 1)


def _quantize(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return to_bf16_bits(x)
    return x.astype(np.float32)


def _draft_tokens(zq_stored: np.ndarray, dtype: str) -> np.ndarray:
    vals = bf16_bits_to_float(zq_stored) if dtype == "bf16" else zq_stored
    return np.argmax(vals, axis=1).astype(np.int32)


def _gen_request(c: dict, seed: int, b: int, n_rows: int):
    rng = _stream(seed, c["cid"], 0, b)
    sig = _request_sigma(c, rng, n_rows)
    V = c["V"]
    zp = rng.normal(0.0, TARGET_STD, size=(n_rows, V))
    peaks = rng.integers(0, V, size=n_rows)
    zp[np.arange(n_rows), peaks] += PEAK
    noise = rng.normal(0.0, 1.0, size=(n_rows, V))
    zq = zp + noise * sig[:, None]
    zp_s = _quantize(zp, c["dtype"])
    zq_s = _quantize(zq, c["dtype"])
    return zp_s, zq_s, _draft_tokens(zq_s, c["dtype"])


def _sigma_of_request(c: dict, seed: int, b: int) -> float:
    rng = _stream(seed, c["cid"], 0, b)
    return float(_request_sigma(c, rng, 1)[0])


def _ragged_lengths(c: dict, seed: int) -> np.ndarray:
    k, B = c["k"], c["B"]
    p = 1.0 / np.arange(1, k + 1, dtype=np.float64)
    p /= p.sum()
    rng = _stream(seed, c["cid"], 2)
    return (rng.choice(k, size=B, p=p) + 1).astype(np.int32)


def _head_inputs(c: dict, seed: int):
    B, H = c["B"], c["H"]
    rng = _stream(seed, c["cid"], 1)
    sd = 1.0 / math.sqrt(H)
    w = rng.normal(0.0, sd, size=H)
    h = rng.normal(0.0, sd, size=(B, H))
    if c["bk"] == "planted":
        ww = float(np.dot(w, w))
        for b in range(B):
            s = _sigma_of_request(c, seed, b)
            t = min(max((4.0 - s) / 3.7, 1e-3), 1.0 - 1e-3)
            target = math.log(t / (1.0 - t))
            h[b] = h[b] + (target - float(np.dot(w, h[b]))) * w / ww
    return h.astype(np.float32), w.astype(np.float32)


def _default_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make(name: str, seed: int = 0, workers: Optional[int] = None, **overrides) -> Workload:
    """Build a whole workload.  Overrides (B, k, V, H, dtype, sigma, lam, tau,
    ...) give smaller or edge-case variants of the same recipe.  Requests are
    generated on `workers` threads; each request has its own random stream,
    so the result does not depend on the thread count."""
    c = _cfg(name, overrides)
    B, k, V = c["B"], c["k"], c["V"]
    if c["layout"] == "ragged":
        n = _ragged_lengths(c, seed)
        row_off = np.zeros(B + 1, dtype=np.int32)
        row_off[1:] = np.cumsum(n)
    else:
        n = np.full(B, k, dtype=np.int32)
        row_off = None
    R = int(n.sum())
    sdt = np.uint16 if c["dtype"] == "bf16" else np.float32
    zp = np.empty((R, V), dtype=sdt)
    zq = np.empty((R, V), dtype=sdt)
    draft = np.empty(R, dtype=np.int32)
    starts = np.concatenate([[0], np.cumsum(n)[:-1]]).astype(np.int64)

    def fill(b: int) -> None:
        p_s, q_s, d = _gen_request(c, seed, b, int(n[b]))
        r0 = int(starts[b])
        zp[r0:r0 + n[b]] = p_s
        zq[r0:r0 + n[b]] = q_s
        draft[r0:r0 + n[b]] = d

    nw = workers or _default_workers()
    if nw <= 1 or B == 1:
        for b in range(B):
            fill(b)
    else:
        with concurrent.futures.ThreadPoolExecutor(max_workers=nw) as ex:
            list(ex.map(fill, range(B)))
    if c["bk"] in ("head", "planted"):
        h, w = _head_inputs(c, seed)
    else:
        h = w = None
    return Workload(name=name, seed=seed, dtype=c["dtype"], B=B, k=k, V=V, H=c["H"],
                    layout=c["layout"], lam=float(c["lam"]), tau=float(c["tau"]),
                    gamma=1.0, round_mode="ceil", zp=zp, zq=zq, draft=draft,
                    row_off=row_off, h=h, w=w, bias=0.0)


def request_rows(name: str, seed: int, b: int, **overrides):
    """Regenerate only request b's stored rows: (zp, zq, draft).  Identical to
    the corresponding rows of make(name, seed, **overrides)."""
    c = _cfg(name, overrides)
    if c["layout"] == "ragged":
        n = int(_ragged_lengths(c, seed)[b])
    else:
        n = c["k"]
    return _gen_request(c, seed, b, n)
