"""The seeded input generator: number formats, determinism, recipe shape."""

import numpy as np
import torch

import oracle
import synth


def test_bf16_rounding_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.normal(0, 4, 200000), rng.normal(0, 1e-3, 1000), rng.normal(0, 1e4, 1000)])
    x32 = x.astype(np.float32)
    ours = synth.to_bf16_bits(x32.astype(np.float64))
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_rounding_is_single_rounding_from_float64():
    # 1 + 2^-8 is the midpoint between bf16 neighbours 1 and 1 + 2^-7; a value
    # just above it must round up, although rounding to float32 first would
    # land exactly on the midpoint and then tie to the even neighbour 1.0.
    x = np.array([1 + 2.0 ** -8 + 2.0 ** -30, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8 + 2.0 ** -30)])
    got = synth.bf16_bits_to_float(synth.to_bf16_bits(x)).astype(np.float64)
    assert list(got) == [1 + 2.0 ** -7, 1.0, 1 + 2 * 2.0 ** -7, -(1 + 2.0 ** -7)]


def test_generation_is_deterministic_and_request_rows_agree():
    a = synth.make("concurrent", seed=3, B=4, V=1000)
    b = synth.make("concurrent", seed=3, B=4, V=1000)
    assert np.array_equal(a.zp, b.zp) and np.array_equal(a.zq, b.zq)
    assert np.array_equal(a.h, b.h)
    zp2, zq2, d2 = synth.request_rows("concurrent", 3, 2, B=4, V=1000)
    r0, n = a.rows_of(2)
    assert np.array_equal(zp2, a.zp[r0:r0 + n]) and np.array_equal(d2, a.draft[r0:r0 + n])
    c = synth.make("concurrent", seed=4, B=4, V=1000)
    assert not np.array_equal(a.zp, c.zp)


def test_draft_tokens_are_first_argmax_of_stored_drafter_logits():
    w = synth.make("single", V=3000)
    vals = synth.bf16_bits_to_float(w.zq)
    assert np.array_equal(w.draft, np.argmax(vals, axis=1))
    t = synth.make("tiny")
    assert t.zp.dtype == np.float32 and np.array_equal(t.draft, np.argmax(t.zq, axis=1))


def test_noise_ramp_and_peak():
    w = synth.make("tiny", V=20000)
    d = (w.zq.astype(np.float64) - w.zp.astype(np.float64)).std(axis=1)
    ramp = 0.5 + 2.5 * np.arange(16) / 15
    np.testing.assert_allclose(d, ramp, rtol=0.05)
    zp = w.zp.astype(np.float64)
    assert abs(zp.std() - 2.0) < 0.05
    assert np.all(zp.max(axis=1) > 5.0)


def test_ragged_lengths_and_layout():
    w = synth.make("ragged", V=64)
    n = np.diff(w.row_off)
    assert w.row_off[0] == 0 and w.R == w.row_off[-1]
    assert n.min() >= 1 and n.max() <= 16
    # p(b) proportional to 1/b favours short blocks: E[b] = 16 / H_16 ~ 4.73
    assert 3.5 < n.mean() < 6.0
    assert np.count_nonzero(n == 1) > np.count_nonzero(n == 16)


def test_planted_head_spreads_verification_lengths():
    w = synth.make("concurrent", V=64)
    _, bk, margin = oracle.length_head(w.h, w.w, w.bias, w.gamma, w.k)
    assert len(set(bk.tolist())) >= 12
    assert margin.min() > 1e-9
    # the plain random head of the other workloads clusters at k/2
    t = synth.make("single", V=64)
    _, bk1, _ = oracle.length_head(t.h, t.w, t.bias, t.gamma, t.k)
    assert bk1[0] in (8, 9)
