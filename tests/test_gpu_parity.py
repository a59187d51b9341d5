"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
the same seeded inputs.  Small shapes are compared entry by entry on every
row; the full-size workloads, in the launch configuration the benchmark
uses, are compared on every argmax and acceptance length and on sampled rows
of loss, statistics and gradient."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
import parity_util
from parity_util import (check_workload, gpu_inputs, logits_tensor, oracle_reductions, run_fwd,
                         spans)

# forked processes that run the oracle over every row of a full-size workload
ORACLE_WORKERS = 8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def av():
    import drafter_distillation_amd as dd
    dd.lib()
    return dd


def head_bk(w):
    _, bk, _ = oracle.length_head(w.h, w.w, w.bias, w.gamma, w.k)
    return bk


def say(msg):
    print(msg, flush=True)


def assert_no_errors(errors):
    assert not errors, "\n".join(errors[:10])


# onchip: 0 = automatic; else (vectors per thread in registers) | (in LDS) << 8,
# the rest of the row streamed twice -- small values exercise every path.
ONCHIP = [0, 1, 1 | (1 << 8), 2 | (3 << 8)]


# ---------------------------------------------------------------------------
# length head
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "single", "concurrent", "long"])
@pytest.mark.parametrize("mode", ["ceil", "floor"])
def test_length_head(av, name, mode):
    w = synth.make(name, V=64)  # only the head inputs matter here
    say(f"length head {name} {mode}")
    for gamma, bias in [(1.0, 0.0), (0.75, 0.3), (1.6, -2.0)]:
        rate, bk = av.av_length_head(torch.from_numpy(w.h).cuda(), torch.from_numpy(w.w).cuda(),
                                     bias, gamma, w.k,
                                     av.AV_ROUND_CEIL if mode == "ceil" else av.AV_ROUND_FLOOR)
        ref_rate, ref_bk, margin = oracle.length_head(w.h, w.w, bias, gamma, w.k, mode)
        rate, bk = rate.cpu().numpy(), bk.cpu().numpy()
        # no seeded b_k lies within 1e-9 of a rounding boundary: every one
        # must match bit for bit
        assert margin.min() > 1e-9, margin.min()
        assert np.array_equal(bk, ref_bk)
        np.testing.assert_allclose(rate, ref_rate, rtol=1e-6, atol=1e-30)


@pytest.mark.parametrize("H", [301, 4097, 4096])
def test_length_head_odd_width_and_misaligned(av, H):
    # the dot product reads 16-byte vectors only when H % 4 == 0 and both
    # operands are 16-byte aligned; odd widths and an operand at a 4-byte
    # offset take the scalar loop
    rng = np.random.default_rng(H)
    B = 37
    h = (rng.standard_normal((B, H)) / np.sqrt(H)).astype(np.float32)
    w = (rng.standard_normal(H) / np.sqrt(H) * 8.0).astype(np.float32)
    buf = torch.empty(B * H + 1, dtype=torch.float32, device="cuda")
    hd = buf[1:].view(B, H)
    hd.copy_(torch.from_numpy(h))
    for hh in (torch.from_numpy(h).cuda(), hd):
        rate, bk = av.av_length_head(hh, torch.from_numpy(w).cuda(), 0.1, 1.0, 16)
        ref_rate, ref_bk, margin = oracle.length_head(h, w, 0.1, 1.0, 16)
        rate, bk = rate.cpu().numpy(), bk.cpu().numpy()
        assert margin.min() > 1e-9, margin.min()
        assert np.array_equal(bk, ref_bk)
        np.testing.assert_allclose(rate, ref_rate, rtol=1e-6, atol=1e-30)


def test_length_head_extremes(av):
    H = 300
    w = np.full(H, 1.0, np.float32)
    h = np.stack([np.zeros(H), np.full(H, 0.5), np.full(H, -0.5), np.full(H, 1e-3)]).astype(np.float32)
    for mode, code in (("ceil", av.AV_ROUND_CEIL), ("floor", av.AV_ROUND_FLOOR)):
        rate, bk = av.av_length_head(torch.from_numpy(h).cuda(), torch.from_numpy(w).cuda(),
                                     0.0, 1.0, 16, code)
        _, ref, _ = oracle.length_head(h, w, 0.0, 1.0, 16, mode)
        assert list(bk.cpu().numpy()) == list(ref)
        assert rate.cpu().numpy()[0] == 0.5


# ---------------------------------------------------------------------------
# whole-batch parity on small shapes (every row, every entry)
# ---------------------------------------------------------------------------

def full_parity(av, w, bk, lam, tau, gs=1.0, vecs=0, split=0):
    say(f"parity {w.name} B={w.B} k={w.k} V={w.V} {w.dtype} {w.layout} lam={lam} tau={tau} "
        f"gs={gs} vecs={vecs} split={split}")
    inp = gpu_inputs(w)
    out = run_fwd(av, inp, w, bk=bk, lam=lam, tau=tau, gs=gs, vecs=vecs, split=split)
    assert_no_errors(check_workload(out, w, bk, lam, tau, gs))
    ref = oracle_reductions(w, bk, lam, tau, gs)
    np.testing.assert_allclose(out["req_loss"], ref["req_loss"], rtol=1e-3, atol=1e-4)
    assert math.isclose(out["total_loss"][0], ref["total_loss"], rel_tol=1e-3, abs_tol=1e-4)
    return out


@pytest.mark.parametrize("vecs", ONCHIP)
def test_tiny_workload(av, vecs):
    w = synth.make("tiny")
    full_parity(av, w, head_bk(w), w.lam, w.tau, vecs=vecs)


def test_single_request_full_vocab(av):
    w = synth.make("single")
    full_parity(av, w, head_bk(w), w.lam, w.tau)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [1, 7, 8, 37, 64, 1000, 2056, 10000, 10001, 65544])
@pytest.mark.parametrize("vecs", ONCHIP)
def test_small_shapes(av, dtype, V, vecs):
    w = synth.make("concurrent", B=3, V=V, dtype=dtype)
    bk = np.array([1, 16, 7])
    full_parity(av, w, bk, 0.5, 0.1, gs=0.25, vecs=vecs)


# Rows wide enough for the fast form (every on-chip slot filled: 13 slots of
# 1024 16-byte vectors), at the edges of its LDS ring: no streamed slot, one
# partial streamed slot of a single vector, one full slot, and an odd count
# that ends in a partial slot only some waves load.
FAST_BF16 = [106496, 106496 + 8, 106496 + 8192, 106496 + 2 * 8192 + 512 * 8]
FAST_F32 = [53248, 53248 + 4, 53248 + 2 * 4096 + 100 * 4]


@pytest.mark.parametrize("dtype,V", [("bf16", v) for v in FAST_BF16] + [("f32", v) for v in FAST_F32])
def test_fast_form_ring_edges(av, dtype, V):
    w = synth.make("concurrent", B=3, V=V, dtype=dtype)
    bk = np.array([1, 16, 7])
    out = full_parity(av, w, bk, 0.5, 0.1, gs=0.25)
    inp = gpu_inputs(w)
    g = av.av_verify_opd_bwd(inp["zp"], inp["zq"], torch.from_numpy(out["tgt_argmax"]).cuda(),
                             torch.from_numpy(out["row_stats"]).cuda(), k=w.k, lam=0.5, tau=0.1,
                             grad_scale=0.25, bk=torch.from_numpy(bk.astype(np.int32)).cuda())
    assert np.array_equal(g.cpu().numpy().view(np.uint32), out["grad"].view(np.uint32))


# Split rows (each verified row's halves on two workgroups that exchange
# statistics, a launch form the test hook selects): at small widths (general
# form, the halves partly streamed when the on-chip knob is small), then at
# widths where the halves take the fast form with 5 register slots (halves of
# 9..12 full slots: none, one partial, one full or almost four streamed) or
# with 9 (halves of 13 slots or more).
SPLIT_V = [16, 64, 1000, 10000, 10008, 65544]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", SPLIT_V)
@pytest.mark.parametrize("vecs", [0, 1 | (1 << 8)])
@pytest.mark.parametrize("split", [2, 4])
def test_split_rows_small_shapes(av, dtype, V, vecs, split):
    # split 4 at V = 16 (f32: 4 vectors) leaves three of the four parts empty
    w = synth.make("concurrent", B=3, V=V, dtype=dtype)
    bk = np.array([1, 16, 7])
    full_parity(av, w, bk, 0.5, 0.1, gs=0.25, vecs=vecs, split=split)


SPLIT_FAST_BF16 = [147456, 151936, 163840, 212992 - 8, 212992, 262144]
SPLIT_FAST_F32 = [73728, 73728 + 4 * 100, 106496 + 4 * 4096]


@pytest.mark.parametrize("dtype,V", [("bf16", v) for v in SPLIT_FAST_BF16] + [("f32", v) for v in SPLIT_FAST_F32])
def test_split_rows_fast_forms(av, dtype, V):
    w = synth.make("concurrent", B=2, V=V, dtype=dtype)
    bk = np.array([16, 5])
    out = full_parity(av, w, bk, 0.5, 0.1, gs=0.25, split=2)
    inp = gpu_inputs(w)
    g = av.av_verify_opd_bwd(inp["zp"], inp["zq"], torch.from_numpy(out["tgt_argmax"]).cuda(),
                             torch.from_numpy(out["row_stats"]).cuda(), k=w.k, lam=0.5, tau=0.1,
                             grad_scale=0.25, bk=torch.from_numpy(bk.astype(np.int32)).cuda())
    assert np.array_equal(g.cpu().numpy().view(np.uint32), out["grad"].view(np.uint32))
    # the same rows as whole rows give the same argmax, acceptance and the
    # same losses to rounding
    whole = run_fwd(av, inp, w, bk=bk, lam=0.5, tau=0.1, gs=0.25, split=1)
    assert np.array_equal(whole["tgt_argmax"], out["tgt_argmax"])
    assert np.array_equal(whole["acc_len"], out["acc_len"])
    np.testing.assert_allclose(whole["row_loss"], out["row_loss"], rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("split", [1, 2, 4])
def test_split_rows_ragged_and_ties(av, split):
    w = synth.make("ragged", B=10, V=9000)
    full_parity(av, w, None, 0.5, 0.1, gs=1.0 / w.R, split=split)
    # exact bf16 ties across the parts: the first part's index wins
    w = synth.make("concurrent", B=1, V=12000, dtype="bf16")
    zp = w.zp.copy()
    big = synth.to_bf16_bits(np.array([40.0]))[0]
    # first entry of the second half (64-vector boundary past the middle),
    # also the first entry of the third quarter (quarters: 384, 768, 1152 vectors)
    cut = 768 * 8
    for i, (j1, j2) in enumerate([(cut - 1, cut), (5, cut + 3), (cut, 11999), (0, 11999)]):
        zp[i, j1] = big
        zp[i, j2] = big
    w.zp = zp
    out = full_parity(av, w, np.array([16]), 0.5, 0.1, split=split)
    assert list(out["tgt_argmax"][:4]) == [cut - 1, 5, cut, 0]


@pytest.mark.parametrize("dtype,V", [("bf16", 151936), ("f32", 73728 + 4 * 100), ("bf16", 40000)])
def test_quarter_rows(av, dtype, V):
    """Rows in quarters on teams of four workgroups: oracle parity, the
    backward from the saved statistics bit for bit, and the same argmax,
    acceptance and losses (to rounding) as whole rows."""
    w = synth.make("concurrent", B=2, V=V, dtype=dtype)
    bk = np.array([16, 5])
    out = full_parity(av, w, bk, 0.5, 0.1, gs=0.25, split=4)
    inp = gpu_inputs(w)
    g = av.av_verify_opd_bwd(inp["zp"], inp["zq"], torch.from_numpy(out["tgt_argmax"]).cuda(),
                             torch.from_numpy(out["row_stats"]).cuda(), k=w.k, lam=0.5, tau=0.1,
                             grad_scale=0.25, bk=torch.from_numpy(bk.astype(np.int32)).cuda())
    assert np.array_equal(g.cpu().numpy().view(np.uint32), out["grad"].view(np.uint32))
    whole = run_fwd(av, inp, w, bk=bk, lam=0.5, tau=0.1, gs=0.25, split=1)
    assert np.array_equal(whole["tgt_argmax"], out["tgt_argmax"])
    assert np.array_equal(whole["acc_len"], out["acc_len"])
    np.testing.assert_allclose(whole["row_loss"], out["row_loss"], rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("dtype,V,vecs", [("bf16", 9000, 0), ("bf16", 5000, 1 | (1 << 8)), ("f32", 3001, 0),
                                          ("f32", 4000, 2 | (1 << 8)), ("bf16", 151936, 0),
                                          ("f32", 73728 + 4 * 100, 0)])
def test_split_tail_forced(av, dtype, V, vecs):
    """Split tail forced (half the rows whole, the rest as pairs of halves
    claimed from the dispenser): small widths in the general form, and the
    widths whose halves fill the fast form's slots."""
    w = synth.make("ragged", B=7, V=V, dtype=dtype)
    out = full_parity(av, w, None, 0.5, 0.1, gs=1.0 / w.R, vecs=vecs, split=3)
    whole = run_fwd(av, gpu_inputs(w), w, bk=None, lam=0.5, tau=0.1, gs=1.0 / w.R, vecs=vecs, split=1)
    assert np.array_equal(whole["tgt_argmax"], out["tgt_argmax"])
    assert np.array_equal(whole["acc_len"], out["acc_len"])


def test_split_tail_ties_across_halves(av):
    # exact bf16 ties in tail rows, across the two halves: the first index wins
    w = synth.make("ragged", B=4, V=12000, dtype="bf16")
    zp = w.zp.copy()
    big = synth.to_bf16_bits(np.array([40.0]))[0]
    cut = 768 * 8  # first entry of the second half
    last = w.R - 1  # a row of the split tail (rows R/2 .. R-1)
    zp[last, cut - 1] = big
    zp[last, cut] = big
    w.zp = zp
    out = full_parity(av, w, None, 0.5, 0.1, split=3)
    assert out["tgt_argmax"][last] == cut - 1


@pytest.mark.parametrize("lam", [0.0, 0.5, 1.0])
@pytest.mark.parametrize("tau", [0.01, 0.05, 0.1, 1e9, float("inf")])
def test_lambda_tau_branches(av, lam, tau):
    w = synth.make("long", B=2, V=24000)
    for vecs, split in ((0, 0), (1 | (1 << 8), 0), (0, 2)):
        full_parity(av, w, np.array([32, 17]), lam, tau, vecs=vecs, split=split)


@pytest.mark.parametrize("vecs", ONCHIP)
def test_ragged_small(av, vecs):
    w = synth.make("ragged", B=10, V=5000)
    full_parity(av, w, None, 0.5, 0.1, gs=1.0 / w.R, vecs=vecs)


def test_verification_length_edges_and_acceptance(av):
    # b_k outside [1, k] is clamped; all-accepted, none-accepted and
    # out-of-range drafts.
    w = synth.make("concurrent", B=6, V=2000)
    zp = oracle.bf16_bits_to_f64(w.zp)
    tgt = np.argmax(zp, axis=1).astype(np.int32)
    d = w.draft.copy()
    d[0:16] = tgt[0:16]                 # request 0 accepts everything
    d[16:32] = tgt[16:32]
    d[16] = (tgt[16] + 1) % w.V         # request 1 rejects the first token
    d[32:48] = tgt[32:48]
    d[35] = -5                          # request 2: out-of-range draft
    d[48:64] = tgt[48:64]
    d[50] = w.V                         # request 3: out-of-range draft (= V)
    d[64:80] = tgt[64:80]               # request 4 accepts all but b_k = 0 -> 1
    w.draft = d
    bk = np.array([16, 16, 16, 99, 0, -3])
    out = full_parity(av, w, bk, 0.5, 0.1)
    assert list(out["acc_len"][:5]) == [16, 0, 3, 2, 1]


def test_ties_across_thread_chunk_and_vector_boundaries(av):
    # bf16 exact ties placed so that the lowest index is in a later thread,
    # a later vector, an earlier chunk, or the same 8-wide vector.
    w = synth.make("concurrent", B=1, V=12000, dtype="bf16")
    zp = w.zp.copy()
    big = synth.to_bf16_bits(np.array([40.0]))[0]
    pairs = [(5, 9), (7, 2047), (2048, 4000), (100, 11999), (3, 4), (8191, 8192), (0, 11998),
             (6000, 6001), (2047, 2048), (11990, 11991), (1, 2), (4095, 4096), (123, 4567),
             (10000, 10001), (9, 10), (2, 11999)]
    for i, (j1, j2) in enumerate(pairs):
        zp[i, j1] = big
        zp[i, j2] = big
    zp[15, 50] = big                    # three-way tie
    w.zp = zp
    for vecs in ONCHIP:
        out = full_parity(av, w, np.array([16]), 0.5, 0.1, vecs=vecs)
        assert list(out["tgt_argmax"][:15]) == [min(p) for p in pairs[:15]]
        assert out["tgt_argmax"][15] == 2


def test_negative_clip_branch(av):
    # Target mass concentrated on one token the drafter under-weights gives
    # r_j = q_j log(q_j / p_j) < -tau (never produced by the seeded workloads).
    rng = np.random.default_rng(7)
    B, k, V = 2, 4, 4096
    zp = rng.normal(0, 1, (B * k, V))
    zq = zp + rng.normal(0, 0.5, (B * k, V))
    for r in range(B * k):
        j = 17 * (r + 1) + (2100 if r % 2 else 0)  # odd rows: in the second half when split
        zp[r, j] = 14.0                 # p_j ~ 0.97
        zq[r, j] = 10.5 + 0.3 * r       # q_j ~ 0.3-0.9
    w = synth.make("concurrent", B=B, V=V, dtype="f32")
    w.k = k
    w.zp = zp.astype(np.float32)
    w.zq = zq.astype(np.float32)
    w.draft = np.argmax(w.zq, axis=1).astype(np.int32)
    t = oracle.row_terms(w.zp[0].astype(np.float64), w.zq[0].astype(np.float64), 0.5, 0.1)
    assert t.r.min() < -0.1             # the negative branch is exercised
    full_parity(av, w, np.array([4, 3]), 0.5, 0.1)
    full_parity(av, w, np.array([4, 3]), 0.0, 0.05, vecs=1)
    full_parity(av, w, np.array([4, 3]), 0.5, 0.1, split=2)


def test_rising_and_falling_logit_ramps(av):
    # Logits that climb by 120 along the row (and rows that fall) keep raising
    # each thread's running maxima: the first sweep's sums are rescaled again
    # and again, in the fast form (every on-chip slot filled) and in the
    # streamed one.
    rng = np.random.default_rng(11)
    B, k, V = 2, 4, 60000
    ramp = np.linspace(-60.0, 60.0, V)
    zp = np.empty((B * k, V))
    for r in range(B * k):
        zp[r] = (ramp if r % 2 == 0 else ramp[::-1]) + rng.normal(0, 0.5, V)
    zq = zp + rng.normal(0, 1.0, (B * k, V))
    w = synth.make("concurrent", B=B, V=V, dtype="f32")
    w.k = k
    w.zp = zp.astype(np.float32)
    w.zq = zq.astype(np.float32)
    w.draft = np.argmax(w.zq, axis=1).astype(np.int32)
    for lam, tau, vecs, split in [(0.5, 0.1, 0, 0), (0.0, 1e9, 0, 0), (0.5, 0.1, 1 | (1 << 8), 0),
                                  (0.5, 0.1, 0, 2)]:
        full_parity(av, w, np.array([4, 3]), lam, tau, vecs=vecs, split=split)


# ---------------------------------------------------------------------------
# standalone backward, determinism, device-side status
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,kw", [("concurrent", dict(B=4, V=10000)),
                                      ("concurrent", dict(B=2, V=1001, dtype="f32")),
                                      ("ragged", dict(B=6, V=4096))])
def test_bwd_matches_fused_bits(av, name, kw):
    w = synth.make(name, **kw)
    bk = None if w.row_off is not None else np.array([1, 16, 9, 4][:w.B])
    inp = gpu_inputs(w)
    say(f"bwd vs fused {name} {kw}")
    for lam, tau in [(0.5, 0.1), (0.0, 1e9), (1.0, 0.05)]:
        out = run_fwd(av, inp, w, bk=bk, lam=lam, tau=tau, gs=0.5)
        kwb = dict(k=w.k, lam=lam, tau=tau, grad_scale=0.5)
        if w.row_off is not None:
            kwb["row_off"] = inp["row_off"]
        else:
            kwb["bk"] = torch.from_numpy(bk.astype(np.int32)).cuda()
        g = av.av_verify_opd_bwd(inp["zp"], inp["zq"], torch.from_numpy(out["tgt_argmax"]).cuda(),
                                 torch.from_numpy(out["row_stats"]).cuda(), **kwb)
        g = g.cpu().numpy()
        assert np.array_equal(g.view(np.uint32), out["grad"].view(np.uint32))


def test_repeat_calls_are_bit_identical(av):
    w = synth.make("concurrent", B=8, V=30000)
    bk = head_bk(w)
    inp = gpu_inputs(w)
    a = run_fwd(av, inp, w, bk=bk, lam=0.5, tau=0.1)
    for _ in range(3):
        b = run_fwd(av, inp, w, bk=bk, lam=0.5, tau=0.1)
        for key in ("tgt_argmax", "acc_len", "row_loss", "req_loss", "total_loss", "row_stats",
                    "grad"):
            assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key


def test_forward_only_matches_fused(av):
    w = synth.make("concurrent", B=3, V=9000)
    bk = np.array([5, 16, 1])
    inp = gpu_inputs(w)
    a = run_fwd(av, inp, w, bk=bk, lam=0.5, tau=0.1)
    b = run_fwd(av, inp, w, bk=bk, lam=0.5, tau=0.1, want_grad=False)
    for key in ("tgt_argmax", "acc_len", "row_loss", "req_loss", "total_loss", "row_stats"):
        assert np.array_equal(a[key], b[key]), key


def test_workspace_reuse_across_shapes(av):
    # One workspace, calls of different shapes and layouts in turn: every
    # structure a call keeps in it must ignore what earlier calls left there.
    cases = [(synth.make("concurrent", B=8, V=30000), np.array([16, 1, 8, 3, 16, 5, 2, 9])),
             (synth.make("concurrent", B=2, V=5000, dtype="f32"), np.array([4, 16])),
             (synth.make("ragged", B=9, V=7000), None),
             (synth.make("long", B=3, V=20000), np.array([32, 7, 19])),
             (synth.make("concurrent", B=8, V=30000), np.array([2, 16, 4, 9, 1, 16, 6, 11]))]
    for rep in range(2):
        for w, bk in cases:
            say(f"reuse rep={rep} {w.name} B={w.B} V={w.V} {w.dtype} {w.layout}")
            for vecs in (0, 1 | (1 << 8)):
                out = run_fwd(av, gpu_inputs(w), w, bk=bk, lam=0.5, tau=0.1, vecs=vecs)
                assert_no_errors(check_workload(out, w, bk, 0.5, 0.1))


def test_bad_ragged_offsets_are_reported_not_computed(av):
    w = synth.make("ragged", B=5, V=512)
    inp = gpu_inputs(w)
    bad = w.row_off.copy()
    bad[2] = bad[1]                      # request 1 with zero rows
    inp["row_off"] = torch.from_numpy(bad.astype(np.int32)).cuda()
    out = av.av_verify_opd_fwd(inp["zp"], inp["zq"], inp["draft"], k=w.k, row_off=inp["row_off"],
                               lam=0.5, tau=0.1)
    torch.cuda.synchronize()
    assert int(out["status"].item()) & av.AV_DEV_BAD_OFFSETS
    # the workspace is left ready for the next call
    good = run_fwd(av, gpu_inputs(w), w, bk=None, lam=0.5, tau=0.1)
    assert int(good["status"][0]) == 0


def test_graph_replay(av):
    # Each replay of a captured launch must see a fresh epoch.
    w = synth.make("concurrent", B=4, V=20000)
    bk = torch.from_numpy(head_bk(w).astype(np.int32)).cuda()
    inp = gpu_inputs(w)
    ref = av.av_verify_opd_fwd(inp["zp"], inp["zq"], inp["draft"], k=w.k, bk=bk, lam=0.5, tau=0.1)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in ref.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = av.av_verify_opd_fwd(inp["zp"], inp["zq"], inp["draft"], k=w.k, bk=bk, lam=0.5,
                                   tau=0.1)  # warm-up: allocates the stream's workspace
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        av.av_verify_opd_fwd(inp["zp"], inp["zq"], inp["draft"], k=w.k, bk=bk, lam=0.5, tau=0.1,
                             out=out)
    for _ in range(4):
        for t in out.values():
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for key in ref:
            assert torch.equal(out[key], ref[key]), key


# ---------------------------------------------------------------------------
# full-size workloads in the benchmark's launch configuration
# ---------------------------------------------------------------------------

def sample_rows(w, bk, n_per_kind=6, seed=0):
    rng = np.random.default_rng(seed)
    ver, unv = [], []
    for r0, n, bkb in spans(w, bk):
        ver.extend(range(r0, r0 + bkb))
        unv.extend(range(r0 + bkb, r0 + n))
    rows = list(rng.choice(ver, size=min(n_per_kind, len(ver)), replace=False))
    rows += [ver[0], ver[-1]]
    if unv:
        rows += list(rng.choice(unv, size=min(n_per_kind // 2, len(unv)), replace=False))
    return sorted(set(int(r) for r in rows))


def grad_row_sums_vanish(out, w, bk):
    # softmax shift invariance: each verified gradient row sums to zero
    g = out["grad"]
    sums = np.abs(g.astype(np.float64).sum(axis=1))
    scale = np.abs(g).max(axis=1) + 1e-30
    assert np.all(sums <= 1e-4 * scale * math.sqrt(w.V)), sums.max()


@pytest.fixture(scope="module")
def concurrent_full():
    say("generating concurrent workload (B=128, k=16, V=151936, bf16)")
    return synth.make("concurrent")


def report_ambiguous(label):
    a = parity_util.AMBIGUOUS
    say(f"{label}: {a['entries']} clip-ambiguous entries in {a['rows']} rows")
    a["rows"] = a["entries"] = 0


def test_full_concurrent(av, concurrent_full):
    """Every row of the benchmark workload against the oracle, entry by entry."""
    w = concurrent_full
    bk = head_bk(w)
    say(f"full concurrent: verified rows {int(np.clip(bk, 1, w.k).sum())}")
    rate, bkg = av.av_length_head(torch.from_numpy(w.h).cuda(), torch.from_numpy(w.w).cuda(),
                                  w.bias, w.gamma, w.k)
    assert np.array_equal(bkg.cpu().numpy(), bk)
    inp = gpu_inputs(w)
    out = run_fwd(av, inp, w, bk=bk, lam=w.lam, tau=w.tau, gs=1.0 / bk.sum())
    del inp
    parity_util.AMBIGUOUS.update(rows=0, entries=0)
    assert_no_errors(check_workload(out, w, bk, w.lam, w.tau, 1.0 / bk.sum(), workers=ORACLE_WORKERS))
    report_ambiguous("full concurrent")
    grad_row_sums_vanish(out, w, bk)


@pytest.mark.parametrize("name", ["concurrent", "long", "ragged"])
def test_full_size_fused_grad_matches_bwd_bits(av, name):
    """Every gradient entry of a full-size workload, checked against the
    standalone backward (separate kernel, separate store pattern) bit for bit;
    the oracle checks above cover sampled rows."""
    say(f"full-size fused vs bwd: {name}")
    w = synth.make(name)
    inp = gpu_inputs(w)
    kw = dict(k=w.k, lam=w.lam, tau=w.tau, grad_scale=0.25)
    if w.row_off is not None:
        kw["row_off"] = inp["row_off"]
    else:
        kw["bk"] = torch.from_numpy(head_bk(w).astype(np.int32)).cuda()
    out = av.av_verify_opd_fwd(inp["zp"], inp["zq"], inp["draft"], **kw)
    g = av.av_verify_opd_bwd(inp["zp"], inp["zq"], out["tgt_argmax"], out["row_stats"], **kw)
    torch.cuda.synchronize()
    assert int(out["status"].item()) == 0
    a, b = out["grad"].view(torch.int32), g.view(torch.int32)
    diff = (a != b).nonzero()
    assert diff.numel() == 0, f"{diff.shape[0]} entries differ, first at {diff[:4].tolist()}"


def test_full_ragged(av):
    """Every row of the ragged workload against the oracle, entry by entry."""
    say("generating ragged workload")
    w = synth.make("ragged")
    inp = gpu_inputs(w)
    out = run_fwd(av, inp, w, bk=None, lam=w.lam, tau=w.tau)
    del inp
    parity_util.AMBIGUOUS.update(rows=0, entries=0)
    assert_no_errors(check_workload(out, w, None, w.lam, w.tau, workers=ORACLE_WORKERS))
    report_ambiguous("full ragged")
    grad_row_sums_vanish(out, w, None)


def test_full_long_block_sweep(av):
    say("generating long workload (B=64, k=32, V=262144, bf16)")
    w = synth.make("long")
    bk = head_bk(w)
    inp = gpu_inputs(w)
    for lam in (0.0, 0.5, 1.0):
        for tau in (0.05, 0.1, 1e9):
            say(f"long: lam={lam} tau={tau}")
            out = run_fwd(av, inp, w, bk=bk, lam=lam, tau=tau)
            if lam == 0.5 and tau == 0.1:  # the configuration's own pair: every row
                parity_util.AMBIGUOUS.update(rows=0, entries=0)
                assert_no_errors(check_workload(out, w, bk, lam, tau, workers=ORACLE_WORKERS))
                report_ambiguous("full long lam=0.5 tau=0.1")
            else:
                rows = sample_rows(w, bk, n_per_kind=3, seed=int(lam * 10 + tau * 100) % 1000)
                assert_no_errors(check_workload(out, w, bk, lam, tau, rows=rows))
