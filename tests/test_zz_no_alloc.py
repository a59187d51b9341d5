"""The no-allocation entry point (av_verify_opd_fwd_noalloc) against the
workspace entry point (av_verify_opd_fwd) on the same inputs: identical
outputs, bit for bit, on two calls in a row, the second with a smaller input
(the library-owned workspace keeps the first call's contents), and a clear
error for a shape whose workspace exceeds the library's array."""

import ctypes

import numpy as np
import pytest
import torch

import synth
from parity_util import gpu_inputs

pytestmark = pytest.mark.gpu

KEYS = ("tgt_argmax", "acc_len", "row_loss", "req_loss", "total_loss", "row_stats", "grad", "status")


@pytest.fixture(scope="module")
def av():
    import drafter_distillation_amd as dd
    dd.lib()
    return dd


def outputs(w, dev="cuda"):
    R, V, B = w.R, w.V, w.B
    return {"tgt_argmax": torch.full((R,), -7, dtype=torch.int32, device=dev),
            "acc_len": torch.full((B,), -7, dtype=torch.int32, device=dev),
            "row_loss": torch.full((R,), 7.0, device=dev),
            "req_loss": torch.full((B,), 7.0, device=dev),
            "total_loss": torch.full((1,), 7.0, device=dev),
            "row_stats": torch.full((R, 4), 7.0, device=dev),
            "grad": torch.full((R, V), 7.0, device=dev),
            "status": torch.full((1,), -7, dtype=torch.int32, device=dev)}


def both(av, w, bk):
    inp = gpu_inputs(w)
    kw = dict(k=w.k, lam=w.lam, tau=w.tau, grad_scale=0.5)
    if w.row_off is not None:
        kw["row_off"] = inp["row_off"]
    else:
        kw["bk"] = torch.from_numpy(np.asarray(bk, dtype=np.int32)).cuda()
    ref = av.av_verify_opd_fwd(inp["zp"], inp["zq"], inp["draft"], out=outputs(w), **kw)
    got = av.av_verify_opd_fwd(inp["zp"], inp["zq"], inp["draft"], out=outputs(w), noalloc=True, **kw)
    torch.cuda.synchronize()
    assert int(got["status"].item()) == 0
    for key in KEYS:
        a, b = ref[key], got[key]
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), key


@pytest.mark.parametrize("order", ["large_then_small", "ragged_then_dense", "halves_then_quarters"])
def test_noalloc_matches_workspace_entry_point(av, order):
    print(f"no-alloc entry point: {order}", flush=True)
    if order == "large_then_small":
        big = synth.make("concurrent", B=8, V=151936)
        both(av, big, np.array([16, 1, 8, 3, 16, 5, 2, 9]))
        small = synth.make("concurrent", B=3, V=20000)
        both(av, small, np.array([2, 16, 7]))
    elif order == "halves_then_quarters":
        # 128 rows of 151936 run in halves on 256 CUs, 32 rows in quarters
        halves = synth.make("concurrent", B=8, V=151936, seed=1)
        both(av, halves, np.array([3, 16, 9, 1, 12, 16, 7, 2]))
        quarters = synth.make("concurrent", B=2, V=151936, seed=2)
        both(av, quarters, np.array([16, 6]))
    else:
        rg = synth.make("ragged", B=12, V=30000)
        both(av, rg, None)
        small = synth.make("concurrent", B=2, V=4096, dtype="f32")
        both(av, small, np.array([4, 16]))


def test_noalloc_rejects_shapes_beyond_its_array(av):
    from drafter_distillation_amd import _lib
    lib = _lib.lib()
    cap = int(lib.av_noalloc_max_bytes())
    assert cap == 4 << 20
    # B * k rows whose workspace exceeds the array: refused before any launch
    B, k = 2048, 16
    assert av.av_workspace_bytes(B, k, B * k) > cap
    P = ctypes.c_void_p(0x10000)
    rc = lib.av_verify_opd_fwd_noalloc(1, B, k, 64, B * k, None, P, P, P, P, 0.5, 0.1, 1.0, 1.0,
                                       P, P, P, None, None, None, None, P, 0, None, None)
    assert rc == av.AV_EUNSUPPORTED
