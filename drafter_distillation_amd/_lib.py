"""ctypes binding of libav.so (include/av.h).

Argument marshalling only: every step of the pass runs in the HIP library.
Tensors are torch CUDA (HIP) tensors; their data pointers and the current
torch stream are handed to the C ABI.  If the library has not been built, or a
tensor is not on a GPU, the calls raise instead of falling back to anything.
"""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libav.so")

AV_OK, AV_EINVAL, AV_EUNSUPPORTED, AV_EHIP = 0, -1, -2, -3
AV_F32, AV_BF16 = 0, 1
AV_ROUND_CEIL, AV_ROUND_FLOOR = 0, 1
AV_DEV_TIMEOUT, AV_DEV_BAD_OFFSETS = 1, 2
AV_MAX_K = 64


class AVError(RuntimeError):
    def __init__(self, fn: str, code: int, detail: str = ""):
        self.code = code
        msg = f"{fn} failed: {av_status_str(code)}"
        if detail:
            msg += f" ({detail})"
        super().__init__(msg)


_lib = None
_lib_lock = threading.Lock()

_vp, _i, _f, _d, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double, ctypes.c_size_t
_SIGS = {
    "av_length_head": (_i, [_vp, _vp, _f, _f, _i, _i, _i, _i, _vp, _vp, _vp]),
    "av_head_update_workspace_bytes": (_sz, [_i]),
    "av_length_head_update": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i,
                                   _d, _d, _d, _d, _d, _vp, _vp, _vp, _vp, _sz, _vp]),
    "av_workspace_bytes": (_sz, [_i, _i, _i]),
    "av_workspace_init": (_i, [_vp, _sz, _vp]),
    "av_verify_opd_fwd": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _f, _f, _f, _f,
                               _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _sz, _vp]),
    "av_verify_opd_fwd_noalloc": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _f, _f, _f, _f,
                                       _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp]),
    "av_noalloc_max_bytes": (_sz, []),
    "av_init": (_i, []),
    "av_test_verify_opd_fwd": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _f, _f, _f, _f,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _sz, _i, _i,
                                    _vp]),
    "av_verify_opd_bwd": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f, _f, _f, _f,
                               _vp, _i, _i, _vp]),
    "av_spec_workspace_bytes": (_sz, [_i, _i]),
    "av_spec_verify": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_uint64, _vp, _i,
                            _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "av_lm_head_workspace_bytes": (_sz, [_i, _i, _i]),
    "av_lm_head_bwd": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "av_lm_head_last_error": (ctypes.c_char_p, []),
    "av_status_str": (ctypes.c_char_p, [_i]),
    "av_last_hip_error": (ctypes.c_char_p, []),
}


def lib() -> ctypes.CDLL:
    """Load libav.so (once).  Raises if it has not been built."""
    global _lib
    with _lib_lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m drafter_distillation_amd.build`")
            h = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGS.items():
                fn = getattr(h, name)
                fn.restype = res
                fn.argtypes = args
            _lib = h
    return _lib


def av_status_str(code: int) -> str:
    return lib().av_status_str(int(code)).decode()


def _check(fn: str, code: int) -> None:
    if code != AV_OK:
        detail = lib().av_last_hip_error().decode() if code == AV_EHIP else ""
        raise AVError(fn, code, detail)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need_gpu(name: str, t: torch.Tensor, dtype=None) -> None:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


# ---------------------------------------------------------------------------
# workspace cache: one scratch buffer per (entry point, device, stream).  The
# fused pass's buffer holds state that persists between its calls (a launch
# epoch and counters), so no other entry point may write into it.
# ---------------------------------------------------------------------------

_ws: dict = {}


def av_workspace_bytes(B: int, k: int, R: int) -> int:
    return int(lib().av_workspace_bytes(int(B), int(k), int(R)))


def workspace(dev: torch.device, nbytes: int, kind: str = "fwd") -> torch.Tensor:
    """A workspace of at least nbytes for `kind` calls on the current stream of
    dev ("fwd": zero-initialised once by av_workspace_init, as the fused pass
    requires)."""
    key = (kind, dev.index, torch.cuda.current_stream(dev).cuda_stream)
    buf = _ws.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 1 << 16), dtype=torch.uint8, device=dev)
        if kind == "fwd":
            _check("av_workspace_init", lib().av_workspace_init(_ptr(buf), buf.numel(), _stream(dev)))
        _ws[key] = buf
    return buf


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def av_length_head(h: torch.Tensor, w: torch.Tensor, bias: float, gamma: float, k: int,
                   round_mode: int = AV_ROUND_CEIL, rate_out: Optional[torch.Tensor] = None,
                   bk_out: Optional[torch.Tensor] = None):
    """Length head (see include/av.h).  Returns (rate [B] float32, bk [B] int32)."""
    _need_gpu("h", h, torch.float32)
    _need_gpu("w", w, torch.float32)
    B, H = h.shape
    if w.shape != (H,):
        raise ValueError("w must have shape [H]")
    dev = h.device
    rate = rate_out if rate_out is not None else torch.empty(B, dtype=torch.float32, device=dev)
    bk = bk_out if bk_out is not None else torch.empty(B, dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        rc = lib().av_length_head(_ptr(h), _ptr(w), float(bias), float(gamma), B, H, int(k),
                                  int(round_mode), _ptr(rate), _ptr(bk), _stream(dev))
    _check("av_length_head", rc)
    return rate, bk


def av_head_update_workspace_bytes(B: int) -> int:
    return int(lib().av_head_update_workspace_bytes(int(B)))


def av_length_head_update(h: torch.Tensor, acc: torch.Tensor, bk: torch.Tensor, k: int, *,
                          w: torch.Tensor, bias: torch.Tensor, m_w: torch.Tensor, v_w: torch.Tensor,
                          m_b: torch.Tensor, v_b: torch.Tensor, step: int, lr: float = 2e-4,
                          beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
                          weight_decay: float = 0.01, want_rate: bool = True,
                          want_grad_h: bool = False) -> dict:
    """Online update of the length head (see include/av.h).  w, bias [1], m_w,
    v_w, m_b [1], v_b [1] are float32 GPU tensors updated in place.  Returns
    dict(loss [1], rate [B] or None, grad_h [B, H] or None)."""
    _need_gpu("h", h, torch.float32)
    _need_gpu("acc", acc, torch.int32)
    _need_gpu("bk", bk, torch.int32)
    for name, t in (("w", w), ("bias", bias), ("m_w", m_w), ("v_w", v_w), ("m_b", m_b), ("v_b", v_b)):
        _need_gpu(name, t, torch.float32)
    B, H = h.shape
    if acc.shape != (B,) or bk.shape != (B,):
        raise ValueError("acc and bk must have shape [B]")
    if w.shape != (H,) or m_w.shape != (H,) or v_w.shape != (H,):
        raise ValueError("w, m_w and v_w must have shape [H]")
    if bias.numel() != 1 or m_b.numel() != 1 or v_b.numel() != 1:
        raise ValueError("bias, m_b and v_b must have one element")
    dev = h.device
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    rate = torch.empty(B, dtype=torch.float32, device=dev) if want_rate else None
    grad_h = torch.empty((B, H), dtype=torch.float32, device=dev) if want_grad_h else None
    with torch.cuda.device(dev):
        ws = workspace(dev, av_head_update_workspace_bytes(B), kind="head_update")
        rc = lib().av_length_head_update(
            _ptr(h), _ptr(acc), _ptr(bk), B, H, int(k), _ptr(w), _ptr(bias), _ptr(m_w), _ptr(v_w),
            _ptr(m_b), _ptr(v_b), int(step), float(lr), float(beta1), float(beta2), float(eps),
            float(weight_decay), _ptr(loss), _ptr(rate), _ptr(grad_h), _ptr(ws), ws.numel(),
            _stream(dev))
    _check("av_length_head_update", rc)
    return dict(loss=loss, rate=rate, grad_h=grad_h)


def av_spec_workspace_bytes(B: int, R: int) -> int:
    return int(lib().av_spec_workspace_bytes(int(B), int(R)))


def av_spec_verify(zp: torch.Tensor, zq: torch.Tensor, draft: torch.Tensor, u: torch.Tensor, *, k: int,
                   seed: int, bk: Optional[torch.Tensor] = None, row_off: Optional[torch.Tensor] = None,
                   want_stats: bool = False, stats_in: Optional[torch.Tensor] = None,
                   out: Optional[dict] = None) -> dict:
    """Sampling-based block verification (see include/av.h).  zp, zq [R, V]
    bf16/f32; draft [R] int32; u [R] float32 uniforms; dense layout with bk
    [B] or ragged with row_off [B+1].  stats_in: [R, 2] or [R, 4] float32
    with lse_p, lse_q in its first two columns (e.g. av_verify_opd_fwd's
    row_stats), or None.  Returns dict(acc_len [B], token [B], row_stats
    [R, 2] or None, status [1])."""
    _need_gpu("zp", zp)
    _need_gpu("zq", zq, zp.dtype)
    _need_gpu("draft", draft, torch.int32)
    _need_gpu("u", u, torch.float32)
    if zp.dim() != 2 or zq.shape != zp.shape or draft.shape != (zp.shape[0],) or u.shape != draft.shape:
        raise ValueError("zp, zq must be [R, V], draft and u [R]")
    R, V = zp.shape
    dev = zp.device
    if row_off is not None:
        _need_gpu("row_off", row_off, torch.int32)
        B = row_off.numel() - 1
    else:
        if bk is None:
            raise ValueError("dense layout needs bk")
        _need_gpu("bk", bk, torch.int32)
        B = bk.numel()
    o = dict(out or {})

    def get(name, shape, dtype):
        t = o.get(name)
        if t is None:
            t = torch.empty(shape, dtype=dtype, device=dev)
            o[name] = t
        return t

    stride = 0
    if stats_in is not None:
        _need_gpu("stats_in", stats_in, torch.float32)
        if stats_in.dim() != 2 or stats_in.shape[0] != R or stats_in.shape[1] < 2:
            raise ValueError("stats_in must be [R, >= 2]")
        stride = stats_in.shape[1]
    acc = get("acc_len", (B,), torch.int32)
    token = get("token", (B,), torch.int32)
    stats = get("row_stats", (R, 2), torch.float32) if want_stats else None
    status = get("status", (1,), torch.int32)
    with torch.cuda.device(dev):
        ws = workspace(dev, av_spec_workspace_bytes(B, R), kind="spec")
        rc = lib().av_spec_verify(
            _dtype_code(zp), B, int(k), V, R, _ptr(row_off), _ptr(zp), _ptr(zq), _ptr(draft), _ptr(bk),
            _ptr(u), ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF), _ptr(stats_in), stride, _ptr(acc),
            _ptr(token), _ptr(stats),
            _ptr(status), _ptr(ws), ws.numel(), _stream(dev))
    _check("av_spec_verify", rc)
    return o


def av_lm_head_bwd(dz: torch.Tensor, w: Optional[torch.Tensor], hid: Optional[torch.Tensor], *,
                   want_d_hid: bool = True, want_d_w: bool = True) -> dict:
    """Backward of the drafter's LM head (see include/av.h): dz [R, V], w
    [V, H], hid [R, H] bfloat16 GPU tensors.  Returns dict(d_hid [R, H],
    d_w [V, H]) float32 (None where not wanted)."""
    _need_gpu("dz", dz, torch.bfloat16)
    R, V = dz.shape
    H = None
    if want_d_hid:
        _need_gpu("w", w, torch.bfloat16)
        if w.shape[0] != V:
            raise ValueError("w must be [V, H]")
        H = w.shape[1]
    if want_d_w:
        _need_gpu("hid", hid, torch.bfloat16)
        if hid.shape[0] != R or (H is not None and hid.shape[1] != H):
            raise ValueError("hid must be [R, H]")
        H = hid.shape[1]
    dev = dz.device
    d_hid = torch.empty((R, H), dtype=torch.float32, device=dev) if want_d_hid else None
    d_w = torch.empty((V, H), dtype=torch.float32, device=dev) if want_d_w else None
    with torch.cuda.device(dev):
        nbytes = int(lib().av_lm_head_workspace_bytes(R, V, H))
        ws = workspace(dev, nbytes, kind="lm_head")
        rc = lib().av_lm_head_bwd(R, V, H, _ptr(dz), _ptr(w) if want_d_hid else None,
                                  _ptr(hid) if want_d_w else None, _ptr(d_hid), _ptr(d_w), _ptr(ws),
                                  ws.numel(), _stream(dev))
    if rc == AV_EHIP:
        raise AVError("av_lm_head_bwd", rc, lib().av_lm_head_last_error().decode())
    _check("av_lm_head_bwd", rc)
    return dict(d_hid=d_hid, d_w=d_w)


def _grad_code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return AV_F32
    if dtype == torch.bfloat16:
        return AV_BF16
    raise ValueError(f"gradient must be float32 or bfloat16, got {dtype}")


def _dtype_code(zp: torch.Tensor) -> int:
    if zp.dtype == torch.bfloat16:
        return AV_BF16
    if zp.dtype == torch.float32:
        return AV_F32
    raise ValueError(f"logits must be bfloat16 or float32, got {zp.dtype}")


def av_verify_opd_fwd(zp: torch.Tensor, zq: torch.Tensor, draft: torch.Tensor, *, k: int,
                      bk: Optional[torch.Tensor] = None, row_off: Optional[torch.Tensor] = None,
                      lam: float, tau: float, grad_scale: float = 1.0, want_grad: bool = True,
                      want_stats: bool = True, onchip_limit: int = 0, split_rows: int = 0,
                      grad_dtype: torch.dtype = torch.float32, temperature: float = 1.0,
                      want_lse_q1: Optional[bool] = None,
                      out: Optional[dict] = None, noalloc: bool = False) -> dict:
    """Fused verify + OPD pass (see include/av.h).

    zp, zq: [R, V] bf16/f32; draft: [R] int32; dense layout with bk [B] int32,
    or ragged layout with row_off [B+1] int32.  Returns a dict of output
    tensors (tgt_argmax, acc_len, row_loss, req_loss, total_loss, row_stats,
    grad, status, and lse_q1 when requested); `out` may supply preallocated
    tensors under those names.  grad_dtype: torch.float32 (default) or
    torch.bfloat16 (each entry rounded to nearest-even bfloat16).
    temperature: of the reverse-KL term; want_lse_q1 defaults to
    want_stats and temperature != 1 (the backward needs lse_q1 then).

    onchip_limit and split_rows are test knobs that force a launch form
    (include/av_test.h); with both 0 the public entry point is called.
    noalloc: call av_verify_opd_fwd_noalloc (library-owned workspace; with
    every output supplied in `out`, nothing is allocated).
    """
    _need_gpu("zp", zp)
    _need_gpu("zq", zq, zp.dtype)
    _need_gpu("draft", draft, torch.int32)
    if zp.dim() != 2 or zq.shape != zp.shape or draft.shape != (zp.shape[0],):
        raise ValueError("zp, zq must be [R, V] and draft [R]")
    R, V = zp.shape
    dev = zp.device
    if row_off is not None:
        _need_gpu("row_off", row_off, torch.int32)
        B = row_off.numel() - 1
    else:
        if bk is None:
            raise ValueError("dense layout needs bk")
        _need_gpu("bk", bk, torch.int32)
        B = bk.numel()
    o = dict(out or {})

    def get(name, shape, dtype):
        t = o.get(name)
        if t is None:
            t = torch.empty(shape, dtype=dtype, device=dev)
            o[name] = t
        return t

    tgt = get("tgt_argmax", (R,), torch.int32)
    acc = get("acc_len", (B,), torch.int32)
    row_loss = get("row_loss", (R,), torch.float32)
    req_loss = get("req_loss", (B,), torch.float32)
    total = get("total_loss", (1,), torch.float32)
    stats = get("row_stats", (R, 4), torch.float32) if want_stats else None
    if want_lse_q1 is None:
        want_lse_q1 = want_stats and float(temperature) != 1.0
    lse1 = get("lse_q1", (R,), torch.float32) if want_lse_q1 else None
    grad = get("grad", (R, V), grad_dtype) if want_grad else None
    if grad is not None:
        _need_gpu("grad", grad, grad_dtype)
    status = get("status", (1,), torch.int32)
    args = (_dtype_code(zp), B, int(k), V, R, _ptr(row_off), _ptr(zp), _ptr(zq), _ptr(draft),
            _ptr(bk), float(lam), float(tau), float(grad_scale), float(temperature), _ptr(tgt),
            _ptr(acc), _ptr(row_loss), _ptr(req_loss), _ptr(total), _ptr(stats), _ptr(lse1),
            _ptr(grad), _grad_code(grad_dtype), _ptr(status))
    if noalloc:
        if onchip_limit or split_rows:
            raise ValueError("noalloc takes the automatic launch form")
        with torch.cuda.device(dev):
            rc = lib().av_verify_opd_fwd_noalloc(*args, _stream(dev))
        _check("av_verify_opd_fwd_noalloc", rc)
        return o
    nbytes = av_workspace_bytes(B, k, R) if B >= 1 and R >= 1 else 0
    with torch.cuda.device(dev):
        ws = workspace(dev, nbytes)
        args = args + (_ptr(ws), ws.numel())
        if onchip_limit or split_rows:
            rc = lib().av_test_verify_opd_fwd(*args, int(onchip_limit), int(split_rows), _stream(dev))
        else:
            rc = lib().av_verify_opd_fwd(*args, _stream(dev))
    _check("av_verify_opd_fwd", rc)
    return o


def av_verify_opd_bwd(zp: torch.Tensor, zq: torch.Tensor, tgt_argmax: torch.Tensor,
                      row_stats: torch.Tensor, *, k: int, bk: Optional[torch.Tensor] = None,
                      row_off: Optional[torch.Tensor] = None, lam: float, tau: float,
                      grad_scale: float = 1.0, vecs_per_thread: int = 0,
                      grad: Optional[torch.Tensor] = None,
                      grad_dtype: torch.dtype = torch.float32, temperature: float = 1.0,
                      lse_q1: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gradient alone from saved statistics (see include/av.h); lse_q1 from
    the forward call is required when temperature != 1."""
    _need_gpu("zp", zp)
    _need_gpu("zq", zq, zp.dtype)
    _need_gpu("tgt_argmax", tgt_argmax, torch.int32)
    _need_gpu("row_stats", row_stats, torch.float32)
    if lse_q1 is not None:
        _need_gpu("lse_q1", lse_q1, torch.float32)
        if lse_q1.shape != (zp.shape[0],):
            raise ValueError("lse_q1 must be [R]")
    R, V = zp.shape
    dev = zp.device
    if row_off is not None:
        _need_gpu("row_off", row_off, torch.int32)
        B = row_off.numel() - 1
    else:
        _need_gpu("bk", bk, torch.int32)
        B = bk.numel()
    if grad is None:
        grad = torch.empty((R, V), dtype=grad_dtype, device=dev)
    _need_gpu("grad", grad, grad_dtype)
    with torch.cuda.device(dev):
        rc = lib().av_verify_opd_bwd(
            _dtype_code(zp), B, int(k), V, R, _ptr(row_off), _ptr(zp), _ptr(zq), _ptr(bk),
            _ptr(tgt_argmax), _ptr(row_stats), _ptr(lse_q1), float(lam), float(tau), float(grad_scale),
            float(temperature), _ptr(grad), _grad_code(grad_dtype), int(vecs_per_thread), _stream(dev))
    _check("av_verify_opd_bwd", rc)
    return grad
