"""GPU parity of the tempered pass (reverse-KL temperature T != 1) against the
float64 oracle, through the C ABI.

The reverse-KL term compares softmax(zp / T) with softmax(zq / T) and the
cross-entropy keeps the plain softmax of zq; the acceptance rule is that of
the plain pass (parity_util) with the gradient's rounding term scaled for T.
Also: T = 1 gives the plain pass's bits; the standalone backward reproduces
the fused gradient bit for bit from the saved statistics and lse_q1; the
bfloat16 gradient is the float32 one rounded to nearest even.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import check_workload, gpu_inputs, oracle_reductions, run_fwd, spans

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def av():
    import drafter_distillation_amd as dd
    dd.lib()
    return dd


def say(msg):
    print(msg, flush=True)


def head_bk(w):
    _, bk, _ = oracle.length_head(w.h, w.w, w.bias, w.gamma, w.k)
    return bk


def parity(av, w, bk, lam, tau, T, gs=1.0, vecs=0, rows=None, inp=None, split=0):
    say(f"tempered parity {w.name} B={w.B} k={w.k} V={w.V} {w.dtype} {w.layout} T={T} lam={lam} "
        f"tau={tau} vecs={vecs} split={split}")
    inp = inp or gpu_inputs(w)
    out = run_fwd(av, inp, w, bk=bk, lam=lam, tau=tau, gs=gs, vecs=vecs, temperature=T, split=split)
    assert out.get("lse_q1") is not None
    errors = check_workload(out, w, bk, lam, tau, gs, rows=rows, temperature=T)
    assert not errors, "\n".join(errors[:10])
    return out


def sample_rows(w, bk, n=6, seed=0):
    rng = np.random.default_rng(seed)
    ver, unv = [], []
    for r0, cnt, bkb in spans(w, bk):
        ver.extend(range(r0, r0 + bkb))
        unv.extend(range(r0 + bkb, r0 + cnt))
    rows = list(rng.choice(ver, size=min(n, len(ver)), replace=False)) + [ver[0], ver[-1]]
    if unv:
        rows += list(rng.choice(unv, size=min(n // 2, len(unv)), replace=False))
    return sorted(set(int(r) for r in rows))


@pytest.mark.parametrize("T", [0.5, 2.0])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [1, 37, 1000, 10001, 65544])
@pytest.mark.parametrize("vecs", [0, 1 | (1 << 8)])
def test_small_shapes(av, T, dtype, V, vecs):
    w = synth.make("concurrent", B=3, V=V, dtype=dtype)
    bk = np.array([1, 16, 7])
    out = parity(av, w, bk, 0.5, 0.05, T, gs=0.5, vecs=vecs)
    ref = oracle_reductions(w, bk, 0.5, 0.05, 0.5, temperature=T)
    np.testing.assert_allclose(out["req_loss"], ref["req_loss"], rtol=1e-3, atol=1e-4)


@pytest.mark.parametrize("T", [0.5, 2.0])
@pytest.mark.parametrize("name,kw,split", [
    ("concurrent", dict(B=2, V=151936), 2),   # rows in halves, fast form with 5 register slots
    ("concurrent", dict(B=2, V=151936), 4),   # rows in quarters
    ("concurrent", dict(B=2, V=40000), 4),    # quarters, general form, some slots streamed
    ("ragged", dict(B=10, V=9000), 3),        # split tail: half the rows whole, the rest in halves
])
def test_split_forms(av, T, name, kw, split):
    """Rows in parts exchange the tempered statistics (and the plain log-sum-exp
    of zq) through the workspace: oracle parity, and the standalone backward
    reproduces the gradient bit for bit from what the pass saved."""
    w = synth.make(name, **kw)
    bk = None if w.row_off is not None else np.array([16, 5])
    inp = gpu_inputs(w)
    out = parity(av, w, bk, 0.5, 0.1, T, gs=0.25, inp=inp, split=split)
    kwb = dict(k=w.k, lam=0.5, tau=0.1, grad_scale=0.25, temperature=T,
               lse_q1=torch.from_numpy(out["lse_q1"]).cuda())
    if w.row_off is not None:
        kwb["row_off"] = inp["row_off"]
    else:
        kwb["bk"] = torch.from_numpy(bk.astype(np.int32)).cuda()
    g = av.av_verify_opd_bwd(inp["zp"], inp["zq"], torch.from_numpy(out["tgt_argmax"]).cuda(),
                             torch.from_numpy(out["row_stats"]).cuda(), **kwb)
    torch.cuda.synchronize()
    assert np.array_equal(g.cpu().numpy().view(np.uint32), out["grad"].view(np.uint32))


@pytest.mark.parametrize("T", [0.25, 0.7, 3.0])
@pytest.mark.parametrize("lam,tau", [(0.0, 0.05), (1.0, 0.05), (0.5, float("inf")), (0.3, 0.002)])
def test_lambda_tau_branches(av, T, lam, tau):
    w = synth.make("long", B=2, V=24000)
    parity(av, w, np.array([32, 5]), lam, tau, T)


@pytest.mark.parametrize("vecs", [0, 2 | (3 << 8)])
def test_ragged(av, vecs):
    w = synth.make("ragged", B=10, V=5000)
    out = parity(av, w, None, 0.5, 0.05, 1.5, vecs=vecs)
    ref = oracle_reductions(w, None, 0.5, 0.05, temperature=1.5)
    np.testing.assert_allclose(out["req_loss"], ref["req_loss"], rtol=1e-3, atol=1e-4)
    assert math.isclose(out["total_loss"][0], ref["total_loss"], rel_tol=1e-3, abs_tol=1e-4)
    np.testing.assert_allclose(out["lse_q1"], ref["lse_q1"], rtol=2e-6, atol=2e-6)


def test_unit_temperature_is_the_plain_pass(av):
    w = synth.make("concurrent", B=4, V=20000)
    inp = gpu_inputs(w)
    bk = torch.tensor([16, 3, 9, 1], dtype=torch.int32, device="cuda")
    kw = dict(k=w.k, bk=bk, lam=0.5, tau=0.05, grad_scale=0.3)
    a = av.av_verify_opd_fwd(inp["zp"], inp["zq"], inp["draft"], **kw)
    a = {k: v.clone() for k, v in a.items()}
    b = av.av_verify_opd_fwd(inp["zp"], inp["zq"], inp["draft"], temperature=1.0, want_lse_q1=True, **kw)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key
    # at T = 1 the plain lse of zq is the row statistic itself
    assert torch.equal(b["lse_q1"], b["row_stats"][:, 1])


@pytest.mark.parametrize("gdt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("name,kw", [("concurrent", dict(B=4, V=10000)), ("ragged", dict(B=6, V=7000))])
def test_bwd_matches_fused_bits(av, gdt, name, kw):
    w = synth.make(name, **kw)
    inp = gpu_inputs(w)
    args = dict(k=w.k, lam=0.4, tau=0.03, grad_scale=0.5, temperature=0.8)
    if w.row_off is not None:
        args["row_off"] = inp["row_off"]
    else:
        args["bk"] = torch.from_numpy(np.array([16, 2, 9, 5], dtype=np.int32)).cuda()
    out = av.av_verify_opd_fwd(inp["zp"], inp["zq"], inp["draft"], grad_dtype=gdt, **args)
    g = av.av_verify_opd_bwd(inp["zp"], inp["zq"], out["tgt_argmax"], out["row_stats"], grad_dtype=gdt,
                             lse_q1=out["lse_q1"], **args)
    torch.cuda.synchronize()
    assert int(out["status"].item()) == 0
    assert torch.equal(g.view(torch.int16), out["grad"].view(torch.int16))


def test_bf16_gradient_is_the_rounded_f32_gradient(av):
    w = synth.make("concurrent", B=3, V=30000)
    inp = gpu_inputs(w)
    kw = dict(k=w.k, bk=torch.tensor([16, 4, 11], dtype=torch.int32, device="cuda"), lam=0.5, tau=0.05,
              temperature=2.0)
    a = av.av_verify_opd_fwd(inp["zp"], inp["zq"], inp["draft"], **kw)
    a = {k: v.clone() for k, v in a.items()}
    b = av.av_verify_opd_fwd(inp["zp"], inp["zq"], inp["draft"], grad_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    assert torch.equal(b["grad"].view(torch.int16), a["grad"].to(torch.bfloat16).view(torch.int16))
    for key in ("tgt_argmax", "acc_len", "row_loss", "row_stats", "lse_q1"):
        assert torch.equal(a[key], b[key]), key


@pytest.fixture(scope="module")
def concurrent_full():
    say("generating concurrent workload (B=128, k=16, V=151936, bf16)")
    return synth.make("concurrent")


@pytest.mark.parametrize("T", [0.5, 2.0])
def test_full_concurrent(av, concurrent_full, T):
    """Full-size workload in the benchmark's launch configuration: every
    argmax and acceptance length, sampled rows of loss, statistics and
    gradient, zero gradient row sums, and the backward's bits."""
    w = concurrent_full
    bk = head_bk(w)
    gs = 1.0 / bk.sum()
    inp = gpu_inputs(w)
    out = parity(av, w, bk, w.lam, w.tau, T, gs=gs, rows=sample_rows(w, bk, seed=int(T * 10)), inp=inp)
    g = out["grad"].astype(np.float64)
    sums = np.abs(g.sum(axis=1))
    assert np.all(sums <= 1e-4 * (np.abs(g).max(axis=1) + 1e-30) * math.sqrt(w.V))
    del g
    kw = dict(k=w.k, bk=torch.from_numpy(bk.astype(np.int32)).cuda(), lam=w.lam, tau=w.tau, grad_scale=gs,
              temperature=T)
    fused = av.av_verify_opd_fwd(inp["zp"], inp["zq"], inp["draft"], **kw)
    back = av.av_verify_opd_bwd(inp["zp"], inp["zq"], fused["tgt_argmax"], fused["row_stats"],
                                lse_q1=fused["lse_q1"], **kw)
    torch.cuda.synchronize()
    diff = (fused["grad"].view(torch.int32) != back.view(torch.int32)).nonzero()
    assert diff.numel() == 0, f"{diff.shape[0]} entries differ, first at {diff[:4].tolist()}"


def test_full_long(av):
    say("generating long workload (B=64, k=32, V=262144, bf16)")
    w = synth.make("long")
    bk = head_bk(w)
    inp = gpu_inputs(w)
    for T, lam, tau in ((0.6, 0.5, 0.05), (4.0, 0.0, 1e9)):
        parity(av, w, bk, lam, tau, T, rows=sample_rows(w, bk, n=3, seed=int(T * 10)), inp=inp)
