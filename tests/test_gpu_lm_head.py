"""GPU parity of the drafter LM head's backward (through the C ABI) against
the float64 oracle.  bfloat16 inputs are exact in both; the GPU accumulates
in float32, so each entry must lie within 1e-3 of the sum of the absolute
products that form it (the task's relative bar, applied to the scale of the
sum rather than to a result that may cancel)."""

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def av():
    import drafter_distillation_amd as dd
    dd.lib()
    return dd


def say(msg):
    print(msg, flush=True)


def bf16_tensor(shape, seed, scale):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda") * scale).to(torch.bfloat16)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def check(got, ref, scale, what):
    bad = np.abs(got - ref) > 1e-3 * scale + 1e-30
    assert not bad.any(), f"{what}: {int(bad.sum())} entries off"


# (1, 1, 1), (3, 1001, 17), (257, 777, 263): element-wise loads (a dimension
# not a multiple of 8), several tiles with ragged edges; (264, 4104, 520):
# 16-byte loads with checked edge tiles in M and N and a partial last K step;
# (512, 8192, 512): unchecked interior tiles only; (64, 151936, 256): one
# tile of d_hid with the sum over V split over 8 workgroups.
@pytest.mark.parametrize("R,V,H", [(1, 1, 1), (5, 300, 64), (3, 1001, 17), (257, 777, 263), (264, 4104, 520),
                                   (512, 8192, 512), (64, 151936, 256)])
def test_shapes(av, R, V, H):
    say(f"lm head bwd R={R} V={V} H={H}")
    dz = bf16_tensor((R, V), 1, 1e-3)
    w = bf16_tensor((V, H), 2, 0.02)
    hid = bf16_tensor((R, H), 3, 1.0)
    out = av.av_lm_head_bwd(dz, w, hid)
    torch.cuda.synchronize()
    dzh, wh, hh = host(dz), host(w), host(hid)
    ref_h, ref_w = oracle.lm_head_backward(dzh, wh, hh)
    check(host(out["d_hid"]), ref_h, np.abs(dzh) @ np.abs(wh), "d_hid")
    check(host(out["d_w"]), ref_w, np.abs(dzh).T @ np.abs(hh), "d_w")


def raw_call(av, dz, w, hid, d_hid, d_w, ws):
    from drafter_distillation_amd import _lib
    R, V = dz.shape
    H = (w if w is not None else hid).shape[1]
    rc = _lib.lib().av_lm_head_bwd(R, V, H, _lib._ptr(dz), _lib._ptr(w), _lib._ptr(hid), _lib._ptr(d_hid),
                                   _lib._ptr(d_w), _lib._ptr(ws), 0 if ws is None else ws.numel(),
                                   _lib._stream(dz.device))
    assert rc == 0, rc


@pytest.mark.parametrize("R,V,H", [(64, 151936, 256), (40, 20000, 300)])
def test_split_sum_and_workspace(av, R, V, H):
    """d_hid with the sum over V split (the workspace the library asks for)
    and in one piece (no workspace): both within the bar of the oracle, and
    repeated calls bit-identical."""
    from drafter_distillation_amd import _lib
    say(f"lm head bwd split sum R={R} V={V} H={H}")
    nbytes = int(_lib.lib().av_lm_head_workspace_bytes(R, V, H))
    assert nbytes > 0
    dz = bf16_tensor((R, V), 11, 1e-3)
    w = bf16_tensor((V, H), 12, 0.02)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    outs = []
    for wsp in (ws, ws, None):
        d_hid = torch.full((R, H), float("nan"), device="cuda")
        raw_call(av, dz, w, None, d_hid, None, wsp)
        outs.append(d_hid)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    dzh, wh = host(dz), host(w)
    ref = dzh @ wh
    scale = np.abs(dzh) @ np.abs(wh)
    check(host(outs[0]), ref, scale, "d_hid split")
    check(host(outs[2]), ref, scale, "d_hid whole")


@pytest.mark.parametrize("n,H", [(264, 520), (512, 256)])
def test_identity_routes_every_entry(av, n, H):
    """dz = I (n x n) makes d_hid = W and d_W = hid exactly (one nonzero
    product per entry, small integers exact in bfloat16): any misrouted
    load, swizzle or transposed read shows as a wrong entry."""
    say(f"lm head bwd identity n={n} H={H}")
    dz = torch.eye(n, device="cuda").to(torch.bfloat16)
    v = torch.arange(n, device="cuda", dtype=torch.float32)[:, None]
    h = torch.arange(H, device="cuda", dtype=torch.float32)[None, :]
    w = ((3 * v + h) % 61 - 30).to(torch.bfloat16)
    hid = ((5 * v + 7 * h) % 53 - 26).to(torch.bfloat16)
    out = av.av_lm_head_bwd(dz, w, hid)
    torch.cuda.synchronize()
    assert torch.equal(out["d_hid"], w.float())
    assert torch.equal(out["d_w"], hid.float())


def test_one_output_only(av):
    dz = bf16_tensor((4, 500), 4, 1e-3)
    w = bf16_tensor((500, 32), 5, 0.02)
    hid = bf16_tensor((4, 32), 6, 1.0)
    a = av.av_lm_head_bwd(dz, w, None, want_d_w=False)
    b = av.av_lm_head_bwd(dz, None, hid, want_d_hid=False)
    c = av.av_lm_head_bwd(dz, w, hid)
    torch.cuda.synchronize()
    assert a["d_w"] is None and b["d_hid"] is None
    assert torch.equal(a["d_hid"], c["d_hid"]) and torch.equal(b["d_w"], c["d_w"])


def test_full_size_sampled(av):
    """The concurrent workload's shape: R=2048 rows, V=151936, H=4096."""
    R, V, H = 2048, 151936, 4096
    say("lm head bwd full size")
    dz = bf16_tensor((R, V), 7, 1e-4)
    w = bf16_tensor((V, H), 8, 0.02)
    hid = bf16_tensor((R, H), 9, 1.0)
    out = av.av_lm_head_bwd(dz, w, hid)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    wh = host(w)
    for r in rng.choice(R, 3, replace=False):
        dzr = host(dz[r])
        ref = dzr @ wh
        check(host(out["d_hid"][r]), ref, np.abs(dzr) @ np.abs(wh), f"d_hid row {r}")
    hh = host(hid)
    for v in rng.choice(V, 8, replace=False):
        dzv = host(dz[:, v])
        ref = dzv @ hh
        check(host(out["d_w"][v]), ref, np.abs(dzv) @ np.abs(hh), f"d_w row {v}")
