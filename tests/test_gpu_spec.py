"""GPU parity of sampling-based verification (through the C ABI) against the
float64 oracle.

Acceptance rule.  Integers are compared exactly except where floating point
decides them within its own error:
  * an acceptance test u q(d) < p(d) whose relative margin is below 1e-5
    (float32 lse carries ~1e-6 relative error into p(d) and q(d)) may go
    either way; the oracle then follows the GPU's decision and the rest of
    the block is compared under it;
  * the replacement token must be the oracle's, or a token whose race key
    trails the oracle's winner by no more than the two keys' float32 error
    bounds (4 ((2e-6 (p + q) + 1e-6 r) / E) each).
lse_p and lse_q of verified rows: |gpu - ref| <= 2e-6 |ref| + 2e-6.
"""

import math

import numpy as np
import pytest
import scipy.stats
import torch

import oracle
import synth
from parity_util import decode_rows, gpu_inputs

pytestmark = pytest.mark.gpu

AMBIG = 1e-5


@pytest.fixture(scope="module")
def av():
    import drafter_distillation_amd as dd
    dd.lib()
    return dd


def say(msg):
    print(msg, flush=True)


def spans(w, bk):
    if w.row_off is not None:
        return [(int(w.row_off[b]), int(w.row_off[b + 1] - w.row_off[b])) for b in range(w.B)]
    return [(b * w.k, min(max(int(bk[b]), 1), w.k)) for b in range(w.B)]


def run_gpu(av, w, bk, u, seed, inp=None, fused_stats=False):
    """fused_stats: take lse_p, lse_q from a fused verify+OPD pass on the same
    inputs (its row_stats, stride 4) instead of the call's own first sweep."""
    inp = inp or gpu_inputs(w)
    kw = dict(k=w.k, seed=seed, want_stats=True)
    if w.row_off is not None:
        kw["row_off"] = inp["row_off"]
    else:
        kw["bk"] = torch.from_numpy(np.asarray(bk, dtype=np.int32)).cuda()
    if fused_stats:
        lay = {key: kw[key] for key in ("row_off", "bk") if key in kw}
        f = av.av_verify_opd_fwd(inp["zp"], inp["zq"], inp["draft"], k=w.k, lam=0.5, tau=0.1, want_grad=False,
                                 **lay)
        kw["stats_in"] = f["row_stats"]
    out = av.av_spec_verify(inp["zp"], inp["zq"], inp["draft"], torch.from_numpy(u).cuda(), **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def key_tol(p, q, r, e):
    return 4.0 * (2e-6 * (p + q) + 1e-6 * r) / e


def check_request(w, b, r0, n, out, u, seed, errors):
    """Compare request b with the oracle, following ambiguous decisions."""
    acc = int(out["acc_len"][b])
    for i in range(min(acc + 1, n)):
        r = r0 + i
        zp, zq = decode_rows(w, "zp", r), decode_rows(w, "zq", r)
        a, margin = oracle.accept_test(zp, zq, int(w.draft[r]), float(u[r]))
        gpu_a = i < acc
        if a != gpu_a and margin > AMBIG:
            errors.append(f"request {b} row {r}: accept {gpu_a} vs oracle {a} (margin {margin:.2e})")
            return
        lp, lq = oracle.opd._logsumexp(zp), oracle.opd._logsumexp(zq)
        st = out["row_stats"][r]
        if abs(st[0] - lp) > 2e-6 * abs(lp) + 2e-6 or abs(st[1] - lq) > 2e-6 * abs(lq) + 2e-6:
            errors.append(f"row {r}: lse ({st[0]}, {st[1]}) vs ({lp}, {lq})")
    tok = int(out["token"][b])
    if acc >= n:
        if tok != -1:
            errors.append(f"request {b}: all accepted but token {tok}")
        return
    r = r0 + acc
    zp, zq = decode_rows(w, "zp", r), decode_rows(w, "zq", r)
    res, key, p, q = oracle.residual_keys(zp, zq, r, seed)
    e = oracle.race_exponentials(r, len(zp), seed)
    best = int(np.argmax(key))
    if tok == best:
        return
    if not 0 <= tok < len(zp):
        errors.append(f"request {b}: token {tok} out of range")
        return
    gap = key[best] - key[tok]
    if gap > key_tol(p[tok], q[tok], res[tok], e[tok]) + key_tol(p[best], q[best], res[best], e[best]):
        errors.append(f"request {b}: token {tok} (key {key[tok]:.6g}) vs oracle {best} (key {key[best]:.6g})")


def check_all(w, bk, out, u, seed, requests=None):
    errors = []
    sp = spans(w, bk)
    for b in (range(w.B) if requests is None else requests):
        r0, n = sp[b]
        check_request(w, b, r0, n, out, u, seed, errors)
        if len(errors) >= 8:
            break
    assert int(out["status"][0]) == 0
    assert not errors, "\n".join(errors)


def sampled_drafts(w, rng):
    """Drafts drawn from the drafter distribution q of each row."""
    d = np.empty(w.R, dtype=np.int32)
    for r in range(w.R):
        zq = decode_rows(w, "zq", r)
        q = np.exp(zq - zq.max())
        d[r] = rng.choice(len(q), p=q / q.sum())
    return d


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [1, 7, 8, 37, 1000, 4100, 65544])
@pytest.mark.parametrize("fused_stats", [False, True])
def test_small_shapes(av, dtype, V, fused_stats):
    w = synth.make("concurrent", B=5, V=V, dtype=dtype)
    rng = np.random.default_rng(V)
    w.draft = sampled_drafts(w, rng)
    bk = np.array([1, 16, 7, 0, 40])
    u = rng.random(w.R).astype(np.float32)
    say(f"spec small {dtype} V={V} fused_stats={fused_stats}")
    for seed in (0, 0xFEDCBA9876543210):
        out = run_gpu(av, w, bk, u, seed, fused_stats=fused_stats)
        check_all(w, bk, out, u, seed)


def test_statistics_input_matches_own_sweep(av):
    """With the fused pass's row statistics given, the call gathers p(d) and
    q(d) instead of sweeping the rows; where both forms get the same lse
    values (the call's own, fed back with stride 2), every output is the
    same bit for bit."""
    w = synth.make("concurrent", B=8, V=20000)
    rng = np.random.default_rng(12)
    w.draft = sampled_drafts(w, rng)
    bk = np.array([16, 1, 5, 9, 16, 2, 7, 12])
    u = rng.random(w.R).astype(np.float32)
    inp = gpu_inputs(w)
    bkt = torch.from_numpy(bk.astype(np.int32)).cuda()
    own = av.av_spec_verify(inp["zp"], inp["zq"], inp["draft"], torch.from_numpy(u).cuda(), k=w.k, seed=4,
                            bk=bkt, want_stats=True)
    fed = av.av_spec_verify(inp["zp"], inp["zq"], inp["draft"], torch.from_numpy(u).cuda(), k=w.k, seed=4,
                            bk=bkt, want_stats=True, stats_in=own["row_stats"].clone())
    torch.cuda.synchronize()
    for key in ("acc_len", "token", "status"):
        assert torch.equal(own[key], fed[key]), key


def test_ragged_and_edge_decisions(av):
    w = synth.make("ragged", B=12, V=3000)
    rng = np.random.default_rng(5)
    w.draft = sampled_drafts(w, rng)
    u = rng.random(w.R).astype(np.float32)
    u[::5] = 0.0            # always accepted when p(d) > 0
    u[1::7] = np.float32(0.99999994)
    w.draft[3] = -1         # out of range: rejected
    w.draft[8] = w.V
    say("spec ragged")
    for fused_stats in (False, True):
        out = run_gpu(av, w, None, u, 11, fused_stats=fused_stats)
        check_all(w, None, out, u, 11)


def test_equal_distributions_accept_everything(av):
    w = synth.make("concurrent", B=4, V=5000)
    w.zq = w.zp.copy()
    u = np.random.default_rng(6).random(w.R).astype(np.float32)
    bk = np.array([16, 3, 1, 9])
    out = run_gpu(av, w, bk, u, 3)
    assert list(out["acc_len"]) == [16, 3, 1, 9]
    assert list(out["token"]) == [-1, -1, -1, -1]


def test_bad_ragged_offsets_are_reported(av):
    w = synth.make("ragged", B=5, V=512)
    inp = gpu_inputs(w)
    bad = w.row_off.copy()
    bad[2] = bad[1]
    inp["row_off"] = torch.from_numpy(bad.astype(np.int32)).cuda()
    u = np.zeros(w.R, np.float32)
    out = av.av_spec_verify(inp["zp"], inp["zq"], inp["draft"], torch.from_numpy(u).cuda(), k=w.k,
                            seed=1, row_off=inp["row_off"])
    torch.cuda.synchronize()
    assert int(out["status"].item()) & av.AV_DEV_BAD_OFFSETS
    assert int(out["acc_len"][1].item()) == 0 and int(out["token"][1].item()) == -1


def test_emitted_tokens_follow_the_target(av):
    """The published theorem on the GPU: drafts from q, acceptance
    min(1, p/q), replacements from the residual -- the emitted token of each
    one-position block is distributed as p."""
    V, B = 6, 20000
    rng = np.random.default_rng(8)
    p = rng.dirichlet(np.ones(V))
    q = rng.dirichlet(np.ones(V))
    zp = np.tile(np.log(p).astype(np.float32), (B, 1))
    zq = np.tile(np.log(q).astype(np.float32), (B, 1))
    draft = rng.choice(V, size=B, p=q).astype(np.int32)
    u = rng.random(B).astype(np.float32)
    out = av.av_spec_verify(torch.from_numpy(zp).cuda(), torch.from_numpy(zq).cuda(),
                            torch.from_numpy(draft).cuda(), torch.from_numpy(u).cuda(), k=1, seed=42,
                            bk=torch.ones(B, dtype=torch.int32).cuda())
    acc = out["acc_len"].cpu().numpy()
    tok = out["token"].cpu().numpy()
    emitted = np.where(acc == 1, draft, tok)
    assert emitted.min() >= 0
    counts = np.bincount(emitted, minlength=V)
    assert scipy.stats.chisquare(counts, p * B).pvalue > 1e-4


def test_repeat_calls_are_identical_and_seeds_matter(av):
    w = synth.make("concurrent", B=8, V=20000)
    rng = np.random.default_rng(9)
    w.draft = sampled_drafts(w, rng)
    bk = np.full(8, 16)
    u = rng.random(w.R).astype(np.float32)
    inp = gpu_inputs(w)
    a = run_gpu(av, w, bk, u, 7, inp)
    b = run_gpu(av, w, bk, u, 7, inp)
    assert np.array_equal(a["acc_len"], b["acc_len"]) and np.array_equal(a["token"], b["token"])
    c = run_gpu(av, w, bk, u, 8, inp)
    assert np.array_equal(a["acc_len"], c["acc_len"])
    rej = a["acc_len"] < 16
    assert rej.any() and not np.array_equal(a["token"][rej], c["token"][rej])


def test_fused_workspace_survives_other_entry_points(av):
    """The fused pass keeps state in its workspace between calls; calls of the
    other entry points on the same stream must leave it intact."""
    w = synth.make("concurrent", B=4, V=3000)
    bk = np.array([16, 2, 9, 5])
    inp = gpu_inputs(w)
    bkt = torch.from_numpy(bk.astype(np.int32)).cuda()
    first = av.av_verify_opd_fwd(inp["zp"], inp["zq"], inp["draft"], k=w.k, bk=bkt, lam=0.5, tau=0.1)
    first = {k: v.clone() for k, v in first.items()}
    u = torch.rand(w.R, device="cuda")
    av.av_spec_verify(inp["zp"], inp["zq"], inp["draft"], u, k=w.k, seed=1, bk=bkt)
    H = 64
    st = dict(w=torch.zeros(H, device="cuda"), bias=torch.zeros(1, device="cuda"),
              m_w=torch.zeros(H, device="cuda"), v_w=torch.zeros(H, device="cuda"),
              m_b=torch.zeros(1, device="cuda"), v_b=torch.zeros(1, device="cuda"))
    av.av_length_head_update(torch.ones((w.B, H), device="cuda"), first["acc_len"], bkt, w.k, step=1, **st)
    again = av.av_verify_opd_fwd(inp["zp"], inp["zq"], inp["draft"], k=w.k, bk=bkt, lam=0.5, tau=0.1)
    torch.cuda.synchronize()
    for key in first:
        assert torch.equal(first[key], again[key]), key


def test_full_concurrent(av):
    say("spec full concurrent (B=128, k=16, V=151936)")
    w = synth.make("concurrent")
    _, bk, _ = oracle.length_head(w.h, w.w, w.bias, w.gamma, w.k)
    rng = np.random.default_rng(10)
    u = rng.random(w.R).astype(np.float32)
    inp = gpu_inputs(w)
    for fused_stats in (False, True):
        out = run_gpu(av, w, bk, u, 0x5EED, inp=inp, fused_stats=fused_stats)
        check_all(w, bk, out, u, 0x5EED)
