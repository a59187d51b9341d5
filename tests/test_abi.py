"""The C ABI on a host without a GPU: the library loads, exports every entry
point include/av.h and include/av_test.h declare, and rejects bad arguments
on the host before it touches the HIP runtime.  No compute call is made
here."""

import ctypes
import os
import re

import pytest

import drafter_distillation_amd as dd
from drafter_distillation_amd import _lib

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = [os.path.join(INCLUDE, n) for n in sorted(os.listdir(INCLUDE)) if n.endswith(".h")]

# Fake device addresses: never dereferenced, because every call below fails
# host-side validation first.  16-byte aligned so only the intended check fails.
P = ctypes.c_void_p(0x10000)
NULL = None


def header_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(av_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = dd.lib()
    names = header_functions()
    assert {"av_length_head", "av_verify_opd_fwd", "av_verify_opd_bwd",
            "av_test_verify_opd_fwd"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    assert dd.av_status_str(0) == "AV_OK"
    assert dd.av_status_str(-1).startswith("AV_EINVAL")
    assert dd.av_status_str(-2).startswith("AV_EUNSUPPORTED")
    assert dd.av_status_str(-3).startswith("AV_EHIP")
    assert "unknown" in dd.av_status_str(7)


def test_workspace_bytes():
    n = dd.av_workspace_bytes(128, 16, 2048)
    assert n % 256 == 0
    assert n >= 2048 * 16 + 128 * 16  # a tagged (argmax, loss) pair per row, a loss sum per request
    assert dd.av_workspace_bytes(128, 16, 2048) == dd.av_workspace_bytes(128, 16, 2048)
    assert dd.av_workspace_bytes(0, 16, 10) == 0
    assert dd.av_workspace_bytes(4, 65, 10) == 0
    assert dd.av_workspace_bytes(4, 16, 65) == 0   # more rows than B*k
    assert dd.av_workspace_bytes(4, 16, 0) == 0


def fwd(**kw):
    a = dict(dtype=1, B=2, k=4, V=64, R=8, row_off=NULL, zp=P, zq=P, draft=P, bk=P, lam=0.5,
             tau=0.1, gs=1.0, temp=1.0, tgt=P, acc=P, row_loss=P, req_loss=NULL, total=NULL, stats=P,
             lse1=NULL, grad=P, gdt=0, status=NULL, ws=P, ws_bytes=1 << 30, vecs=None, split=0,
             stream=NULL)
    a.update(kw)
    args = (a["dtype"], a["B"], a["k"], a["V"], a["R"], a["row_off"], a["zp"], a["zq"], a["draft"],
            a["bk"], a["lam"], a["tau"], a["gs"], a["temp"], a["tgt"], a["acc"], a["row_loss"],
            a["req_loss"], a["total"], a["stats"], a["lse1"], a["grad"], a["gdt"], a["status"], a["ws"],
            a["ws_bytes"])
    if a["vecs"] is None:  # the public entry point
        return _lib.lib().av_verify_opd_fwd(*args, a["stream"])
    return _lib.lib().av_test_verify_opd_fwd(*args, a["vecs"], a["split"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(zp=NULL), dd.AV_EINVAL),
    (dict(zq=NULL), dd.AV_EINVAL),
    (dict(draft=NULL), dd.AV_EINVAL),
    (dict(tgt=NULL), dd.AV_EINVAL),
    (dict(acc=NULL), dd.AV_EINVAL),
    (dict(row_loss=NULL), dd.AV_EINVAL),
    (dict(ws=NULL), dd.AV_EINVAL),
    (dict(bk=NULL), dd.AV_EINVAL),                       # dense needs bk
    (dict(B=0, R=0), dd.AV_EINVAL),
    (dict(k=0), dd.AV_EINVAL),
    (dict(k=65, R=130), dd.AV_EINVAL),
    (dict(V=0), dd.AV_EINVAL),
    (dict(R=9), dd.AV_EINVAL),                           # dense: R must be B*k
    (dict(row_off=P, R=1), dd.AV_EINVAL),               # ragged: R >= B
    (dict(row_off=P, R=9), dd.AV_EINVAL),               # ragged: R <= B*k
    (dict(lam=-0.1), dd.AV_EINVAL),
    (dict(lam=1.5), dd.AV_EINVAL),
    (dict(lam=float("nan")), dd.AV_EINVAL),
    (dict(tau=0.0), dd.AV_EINVAL),
    (dict(tau=-1.0), dd.AV_EINVAL),
    (dict(tau=float("nan")), dd.AV_EINVAL),
    (dict(gs=float("inf")), dd.AV_EINVAL),
    (dict(gs=float("nan")), dd.AV_EINVAL),
    (dict(temp=0.0), dd.AV_EINVAL),
    (dict(temp=-2.0), dd.AV_EINVAL),
    (dict(temp=float("nan")), dd.AV_EINVAL),
    (dict(temp=float("inf")), dd.AV_EINVAL),
    (dict(ws_bytes=256), dd.AV_EINVAL),                  # workspace too small
    (dict(vecs=-1), dd.AV_EINVAL),                       # test hook: knob out of range
    (dict(vecs=0, split=5), dd.AV_EINVAL),
    (dict(vecs=0, split=-1), dd.AV_EINVAL),
    (dict(vecs=0, split=2, zp=NULL), dd.AV_EINVAL),      # the hook validates as the entry point
    (dict(stats=ctypes.c_void_p(0x10004)), dd.AV_EINVAL),  # row_stats not 16-byte aligned
    (dict(ws=ctypes.c_void_p(0x10008)), dd.AV_EINVAL),
    (dict(dtype=2), dd.AV_EUNSUPPORTED),
    (dict(row_off=P, B=5000, R=5000), dd.AV_EUNSUPPORTED),  # ragged offsets cached on chip
    (dict(B=1 << 16, k=64, R=1 << 22, V=1 << 24), dd.AV_EUNSUPPORTED),  # R*V >= 2^46
    (dict(gdt=3), dd.AV_EUNSUPPORTED),                      # gradient type
])
def test_fwd_rejects_bad_arguments_on_host(kw, code):
    assert fwd(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(h=NULL), dd.AV_EINVAL),
    (dict(w=NULL), dd.AV_EINVAL),
    (dict(bk=NULL), dd.AV_EINVAL),
    (dict(B=0), dd.AV_EINVAL),
    (dict(H=0), dd.AV_EINVAL),
    (dict(k=0), dd.AV_EINVAL),
    (dict(k=65), dd.AV_EINVAL),
    (dict(mode=2), dd.AV_EINVAL),
    (dict(gamma=-1.0), dd.AV_EINVAL),
    (dict(gamma=float("inf")), dd.AV_EINVAL),
    (dict(bias=float("nan")), dd.AV_EINVAL),
])
def test_length_head_rejects_bad_arguments_on_host(kw, code):
    a = dict(h=P, w=P, bias=0.0, gamma=1.0, B=4, H=16, k=16, mode=0, rate=P, bk=P, stream=NULL)
    a.update(kw)
    rc = _lib.lib().av_length_head(a["h"], a["w"], a["bias"], a["gamma"], a["B"], a["H"], a["k"],
                                   a["mode"], a["rate"], a["bk"], a["stream"])
    assert rc == code


@pytest.mark.parametrize("kw,code", [
    (dict(zp=NULL), dd.AV_EINVAL),
    (dict(tgt=NULL), dd.AV_EINVAL),
    (dict(stats=NULL), dd.AV_EINVAL),
    (dict(grad=NULL), dd.AV_EINVAL),
    (dict(bk=NULL), dd.AV_EINVAL),
    (dict(lam=2.0), dd.AV_EINVAL),
    (dict(tau=0.0), dd.AV_EINVAL),
    (dict(R=7), dd.AV_EINVAL),
    (dict(vecs=-2), dd.AV_EINVAL),
    (dict(dtype=5), dd.AV_EUNSUPPORTED),
    (dict(V=64 * 256 * 64 + 8), dd.AV_EUNSUPPORTED),     # more than 64 items per row
    (dict(dtype=0, V=64 * 256 * 32 + 4), dd.AV_EUNSUPPORTED),
    (dict(gdt=2), dd.AV_EUNSUPPORTED),
    (dict(temp=0.0), dd.AV_EINVAL),
    (dict(temp=float("inf")), dd.AV_EINVAL),
    (dict(temp=2.0), dd.AV_EINVAL),                      # tempered: lse_q1 required
    (dict(temp=0.5, lam=0.0), dd.AV_EINVAL),
])
def test_bwd_rejects_bad_arguments_on_host(kw, code):
    a = dict(dtype=1, B=2, k=4, V=64, R=8, row_off=NULL, zp=P, zq=P, bk=P, tgt=P, stats=P,
             lse1=NULL, lam=0.5, tau=0.1, gs=1.0, temp=1.0, grad=P, gdt=0, vecs=0, stream=NULL)
    a.update(kw)
    rc = _lib.lib().av_verify_opd_bwd(a["dtype"], a["B"], a["k"], a["V"], a["R"], a["row_off"],
                                      a["zp"], a["zq"], a["bk"], a["tgt"], a["stats"], a["lse1"],
                                      a["lam"], a["tau"], a["gs"], a["temp"], a["grad"], a["gdt"],
                                      a["vecs"], a["stream"])
    assert rc == code


@pytest.mark.parametrize("kw,code", [
    (dict(h=NULL), dd.AV_EINVAL),
    (dict(acc=NULL), dd.AV_EINVAL),
    (dict(bk=NULL), dd.AV_EINVAL),
    (dict(w=NULL), dd.AV_EINVAL),
    (dict(bias=NULL), dd.AV_EINVAL),
    (dict(m_w=NULL), dd.AV_EINVAL),
    (dict(v_b=NULL), dd.AV_EINVAL),
    (dict(ws=NULL), dd.AV_EINVAL),
    (dict(B=0), dd.AV_EINVAL),
    (dict(H=0), dd.AV_EINVAL),
    (dict(k=0), dd.AV_EINVAL),
    (dict(k=65), dd.AV_EINVAL),
    (dict(step=0), dd.AV_EINVAL),
    (dict(lr=-1e-4), dd.AV_EINVAL),
    (dict(lr=float("nan")), dd.AV_EINVAL),
    (dict(beta1=1.0), dd.AV_EINVAL),
    (dict(beta2=-0.1), dd.AV_EINVAL),
    (dict(eps=0.0), dd.AV_EINVAL),
    (dict(wd=float("inf")), dd.AV_EINVAL),
    (dict(ws_bytes=8), dd.AV_EINVAL),                      # needs 16 bytes per request
    (dict(ws=ctypes.c_void_p(0x10004)), dd.AV_EINVAL),     # not 8-byte aligned
])
def test_head_update_rejects_bad_arguments_on_host(kw, code):
    a = dict(h=P, acc=P, bk=P, B=4, H=16, k=16, w=P, bias=P, m_w=P, v_w=P, m_b=P, v_b=P, step=1,
             lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01, loss=NULL, rate=NULL, gh=NULL,
             ws=P, ws_bytes=1 << 20, stream=NULL)
    a.update(kw)
    rc = _lib.lib().av_length_head_update(
        a["h"], a["acc"], a["bk"], a["B"], a["H"], a["k"], a["w"], a["bias"], a["m_w"], a["v_w"],
        a["m_b"], a["v_b"], a["step"], a["lr"], a["beta1"], a["beta2"], a["eps"], a["wd"], a["loss"],
        a["rate"], a["gh"], a["ws"], a["ws_bytes"], a["stream"])
    assert rc == code


@pytest.mark.parametrize("kw,code", [
    (dict(zp=NULL), dd.AV_EINVAL),
    (dict(draft=NULL), dd.AV_EINVAL),
    (dict(u=NULL), dd.AV_EINVAL),
    (dict(acc=NULL), dd.AV_EINVAL),
    (dict(token=NULL), dd.AV_EINVAL),
    (dict(ws=NULL), dd.AV_EINVAL),
    (dict(bk=NULL), dd.AV_EINVAL),
    (dict(B=0), dd.AV_EINVAL),
    (dict(k=65), dd.AV_EINVAL),
    (dict(R=7), dd.AV_EINVAL),
    (dict(ws_bytes=16 * 8 + 2 * 64 * 16 - 1), dd.AV_EINVAL),
    (dict(ws=ctypes.c_void_p(0x10008)), dd.AV_EINVAL),
    (dict(dtype=5), dd.AV_EUNSUPPORTED),
    (dict(sin=P, sstride=1), dd.AV_EINVAL),              # statistics given with a short stride
])
def test_spec_rejects_bad_arguments_on_host(kw, code):
    a = dict(dtype=1, B=2, k=4, V=64, R=8, row_off=NULL, zp=P, zq=P, draft=P, bk=P, u=P, seed=1,
             sin=NULL, sstride=0, acc=P, token=P, stats=NULL, status=NULL, ws=P, ws_bytes=1 << 20, stream=NULL)
    a.update(kw)
    rc = _lib.lib().av_spec_verify(a["dtype"], a["B"], a["k"], a["V"], a["R"], a["row_off"], a["zp"],
                                   a["zq"], a["draft"], a["bk"], a["u"], a["seed"], a["sin"], a["sstride"],
                                   a["acc"], a["token"], a["stats"], a["status"], a["ws"], a["ws_bytes"],
                                   a["stream"])
    assert rc == code


@pytest.mark.parametrize("kw,code", [
    (dict(dz=NULL), dd.AV_EINVAL),
    (dict(R=0), dd.AV_EINVAL),
    (dict(V=0), dd.AV_EINVAL),
    (dict(H=0), dd.AV_EINVAL),
    (dict(w=NULL), dd.AV_EINVAL),        # d_hid wanted without its operand
    (dict(hid=NULL), dd.AV_EINVAL),      # d_w wanted without its operand
    (dict(ws=NULL), dd.AV_EINVAL),       # workspace bytes without a workspace
])
def test_lm_head_rejects_bad_arguments_on_host(kw, code):
    a = dict(R=4, V=64, H=16, dz=P, w=P, hid=P, d_hid=P, d_w=P, ws=P, ws_bytes=1 << 20, stream=NULL)
    a.update(kw)
    rc = _lib.lib().av_lm_head_bwd(a["R"], a["V"], a["H"], a["dz"], a["w"], a["hid"], a["d_hid"],
                                   a["d_w"], a["ws"], a["ws_bytes"], a["stream"])
    assert rc == code


def test_head_update_workspace_bytes():
    assert dd.av_head_update_workspace_bytes(128) == 128 * 16
    assert dd.av_head_update_workspace_bytes(0) == 0


def test_workspace_init_rejects_bad_arguments():
    lib = _lib.lib()
    assert lib.av_workspace_init(NULL, 1 << 20, NULL) == dd.AV_EINVAL
    assert lib.av_workspace_init(P, 16, NULL) == dd.AV_EINVAL
    assert lib.av_workspace_init(ctypes.c_void_p(0x10008), 1 << 20, NULL) == dd.AV_EINVAL


def test_binding_refuses_cpu_tensors():
    import torch
    z = torch.zeros(4, 8)
    with pytest.raises(ValueError):
        dd.av_verify_opd_fwd(z, z, torch.zeros(4, dtype=torch.int32), k=4,
                             bk=torch.ones(1, dtype=torch.int32), lam=0.5, tau=0.1)
