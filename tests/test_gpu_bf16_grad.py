"""bfloat16 gradient output of the fused pass and of the standalone backward.

The bfloat16 gradient is defined as the float32 gradient rounded to nearest
(ties to even).  It is checked against the float64 oracle's gradient, entry
by entry within the float32 bar plus one bfloat16 spacing; and, as a second
check, bit for bit against the float32 result of the same call rounded by
torch.  Every other output must be identical to the float32 call's."""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import decode_rows, gpu_inputs, grad_row_ok_bf16, spans

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def av():
    import drafter_distillation_amd as dd
    dd.lib()
    return dd


def bits(t):
    return t.contiguous().view(torch.int16)


def compare(av, w, bk, vecs=0, lam=0.5, tau=0.1, gs=0.5, every=1, split=0):
    inp = gpu_inputs(w)
    kw = dict(k=w.k, lam=lam, tau=tau, grad_scale=gs, onchip_limit=vecs, split_rows=split)
    if w.row_off is not None:
        kw["row_off"] = inp["row_off"]
    else:
        kw["bk"] = torch.from_numpy(np.asarray(bk, dtype=np.int32)).cuda()
    a = av.av_verify_opd_fwd(inp["zp"], inp["zq"], inp["draft"], **kw)
    b = av.av_verify_opd_fwd(inp["zp"], inp["zq"], inp["draft"], grad_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    assert b["grad"].dtype == torch.bfloat16
    # against the oracle: every verified row, entry by entry
    g = b["grad"].float().cpu().numpy()
    for r0, n, bkb in spans(w, bk):
        for r in range(r0, r0 + bkb):
            if r % every:
                continue
            t = oracle.row_terms(decode_rows(w, "zp", r), decode_rows(w, "zq", r), lam, tau, gs)
            ok = grad_row_ok_bf16(g[r], t, gs)
            assert ok.all(), (r, int(np.argmin(ok)), g[r][np.argmin(ok)], t.grad[np.argmin(ok)])
        assert not g[r0 + bkb:r0 + n].any()
    # and against the float32 call rounded by torch, bit for bit
    assert torch.equal(bits(b["grad"]), bits(a["grad"].to(torch.bfloat16)))
    for key in ("tgt_argmax", "acc_len", "row_loss", "req_loss", "total_loss", "row_stats", "status"):
        assert torch.equal(a[key], b[key]), key
    # the standalone backward writes the same bits
    kwb = {k: v for k, v in kw.items() if k not in ("onchip_limit", "split_rows")}
    g = av.av_verify_opd_bwd(inp["zp"], inp["zq"], b["tgt_argmax"], b["row_stats"],
                             grad_dtype=torch.bfloat16, **kwb)
    torch.cuda.synchronize()
    assert torch.equal(bits(g), bits(b["grad"]))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [1, 7, 8, 37, 1000, 10001, 65544])
@pytest.mark.parametrize("vecs", [0, 1 | (1 << 8)])
def test_small_shapes(av, dtype, V, vecs):
    w = synth.make("concurrent", B=3, V=V, dtype=dtype)
    compare(av, w, np.array([1, 16, 7]), vecs=vecs)


def test_ragged(av):
    compare(av, synth.make("ragged", B=10, V=5000), None)


@pytest.mark.parametrize("name,kw,split", [
    ("concurrent", dict(B=2, V=151936), 2),
    ("concurrent", dict(B=2, V=151936), 4),
    ("ragged", dict(B=10, V=9000), 3),
])
def test_split_forms(av, name, kw, split):
    """Rows in halves or quarters write the bfloat16 gradient of their part."""
    w = synth.make(name, **kw)
    compare(av, w, None if w.row_off is not None else np.array([16, 5]), split=split)


def test_full_concurrent(av):
    w = synth.make("concurrent")
    from oracle import length_head
    _, bk, _ = length_head(w.h, w.w, w.bias, w.gamma, w.k)
    compare(av, w, bk, gs=1.0 / bk.sum(), every=8)  # oracle on every 8th row
