"""GPU parity of the length head's online update (through the C ABI) against
the float64 oracle, on the concurrent workload's head inputs and on small
and ragged shapes.

Acceptance rule: the update computes in float64 and stores float32, so each
float32 output must match the oracle's float64 value (computed from the same
float32 inputs) to within its own rounding: |gpu - ref| <= 2.5e-7 |ref| +
1e-30 (half an ulp is 6e-8 relative; float64 summation order adds ~1e-15).
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

RTOL, ATOL = 2.5e-7, 1e-30


@pytest.fixture(scope="module")
def av():
    import drafter_distillation_amd as dd
    dd.lib()
    return dd


def say(msg):
    print(msg, flush=True)


def close(gpu, ref, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bad = np.abs(gpu - ref) > RTOL * np.abs(ref) + ATOL
    assert not bad.any(), f"{what}: {int(bad.sum())} entries off, e.g. {gpu[bad].ravel()[:3]} vs {ref[bad].ravel()[:3]}"


def _gpu_state(w, bias, state):
    f = lambda a: torch.tensor(np.asarray(a, dtype=np.float32).reshape(-1), device="cuda")
    return dict(w=f(w), bias=f([bias]), m_w=f(state["m_w"]), v_w=f(state["v_w"]),
                m_b=f([state["m_b"]]), v_b=f([state["v_b"]]))


def _host(t):
    return t.cpu().numpy().astype(np.float64)


def run_steps(av, h, accs, bks, k, w, bias, nsteps=1, want_grad_h=True, **hyper):
    """Runs nsteps updates on the GPU; each is compared with one oracle step
    taken from the GPU's own float32 state before it."""
    H = h.shape[1]
    state = dict(m_w=np.zeros(H), v_w=np.zeros(H), m_b=0.0, v_b=0.0, t=0)
    g = _gpu_state(w, bias, state)
    ht = torch.tensor(h.astype(np.float32), device="cuda")
    hf = h.astype(np.float32).astype(np.float64)
    for step in range(1, nsteps + 1):
        acc, bk = accs[step - 1], bks[step - 1]
        before = dict(w=_host(g["w"]), bias=float(_host(g["bias"])[0]),
                      state=dict(m_w=_host(g["m_w"]), v_w=_host(g["v_w"]), m_b=float(_host(g["m_b"])[0]),
                                 v_b=float(_host(g["v_b"])[0]), t=step - 1))
        out = av.av_length_head_update(ht, torch.tensor(acc, dtype=torch.int32, device="cuda"),
                                       torch.tensor(bk, dtype=torch.int32, device="cuda"), k, step=step,
                                       want_grad_h=want_grad_h, **g, **hyper)
        torch.cuda.synchronize()
        ref = oracle.length_head_update(hf, before["w"], before["bias"], acc, bk, k, before["state"],
                                        **{kk: v for kk, v in hyper.items()})
        close(_host(out["loss"]), [ref["loss"]], "loss")
        if out["rate"] is not None:
            close(_host(out["rate"]), ref["rate"], "rate")
        if want_grad_h:
            close(_host(out["grad_h"]), ref["g_h"], "grad_h")
        close(_host(g["w"]), ref["w"], "w")
        close(_host(g["bias"]), [ref["bias"]], "bias")
        close(_host(g["m_w"]), ref["state"]["m_w"], "m_w")
        close(_host(g["v_w"]), ref["state"]["v_w"], "v_w")
        close(_host(g["m_b"]), [ref["state"]["m_b"]], "m_b")
        close(_host(g["v_b"]), [ref["state"]["v_b"]], "v_b")
    return g


def _accs(rng, bk, n):
    return [np.array([rng.integers(0, b + 1) for b in np.clip(bk, 1, None)]) for _ in range(n)]


def test_concurrent_head_three_steps(av):
    """The concurrent workload's head (B=128, H=4096, k=16), three steps."""
    w = synth.make("concurrent", V=64)  # only the head inputs matter here
    _, bk, _ = oracle.length_head(w.h, w.w, w.bias, w.gamma, w.k)
    rng = np.random.default_rng(0)
    say(f"head update B={w.h.shape[0]} H={w.h.shape[1]}")
    run_steps(av, w.h, _accs(rng, bk, 3), [bk] * 3, w.k, w.w, w.bias, nsteps=3)


# (1, 1), (3, 300), (7, 257): one or a few 64-column workgroups, ragged last
# one; (1500, 70), (5000, 24): more requests than one pass of the step
# kernel's shared-memory chunk of d loss / d z (1024); (128, 5120): 80
# workgroups.
@pytest.mark.parametrize("B,H", [(1, 1), (3, 300), (1500, 70), (7, 257), (128, 5120), (5000, 24)])
def test_shapes(av, B, H):
    rng = np.random.default_rng(B * 1000 + H)
    h = rng.normal(0, 1, (B, H)).astype(np.float32)
    w = rng.normal(0, 1 / math.sqrt(H), H).astype(np.float32)
    bk = rng.integers(1, 17, B)
    say(f"head update shape B={B} H={H}")
    run_steps(av, h, _accs(rng, bk, 2), [bk, bk], 16, w, float(np.float32(0.1)), nsteps=2)


def test_label_edges_and_hyperparameters(av):
    rng = np.random.default_rng(9)
    B, H, k = 6, 40, 16
    h = rng.normal(0, 1, (B, H)).astype(np.float32)
    w = rng.normal(0, 0.2, H).astype(np.float32)
    bk = np.array([16, 9, 0, -3, 99, 4])        # clamps to 16, 9, 1, 1, 16, 4
    acc = np.array([16, 0, 1, 0, 16, 2])
    for hyper in (dict(), dict(weight_decay=0.0), dict(beta1=0.0, beta2=0.0), dict(lr=1e-2, eps=1e-4)):
        run_steps(av, h, [acc], [bk], k, w, -0.3, nsteps=1, want_grad_h=False, **hyper)


def test_exact_prediction_only_decays(av):
    # h = 0, bias = 0: rate 1/2 equals acc / b_k = 4 / 8, so every gradient
    # is zero and the step only applies the weight decay
    B, H, k = 8, 300, 16
    w = np.linspace(-1, 1, H).astype(np.float32)
    g = run_steps(av, np.zeros((B, H), np.float32), [np.full(B, 4)], [np.full(B, 8)], k, w, 0.0)
    ref = (w.astype(np.float64) * (1.0 - 2e-4 * 0.01)).astype(np.float32)
    assert np.array_equal(g["w"].cpu().numpy(), ref)
    assert float(g["bias"].item()) == 0.0
    assert not g["m_w"].any().item() and not g["v_w"].any().item()


def test_graph_replay_matches_eager(av):
    """A captured update, replayed from the same starting state several times
    (with eager work between replays), gives the eager update's bits."""
    rng = np.random.default_rng(11)
    B, H, k = 16, 200, 16
    h = torch.tensor(rng.normal(0, 1, (B, H)).astype(np.float32), device="cuda")
    acc = torch.tensor(rng.integers(0, 9, B), dtype=torch.int32, device="cuda")
    bk = torch.full((B,), 8, dtype=torch.int32, device="cuda")
    init = _gpu_state(rng.normal(0, 0.1, H), 0.2,
                      dict(m_w=rng.normal(0, 1e-3, H), v_w=rng.uniform(0, 1e-6, H), m_b=1e-3, v_b=1e-7))
    st = {n: t.clone() for n, t in init.items()}
    ref = av.av_length_head_update(h, acc, bk, k, step=3, want_grad_h=True, **st)
    torch.cuda.synchronize()
    ref_state = {n: t.clone() for n, t in st.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # allocates this stream's workspace before capture
        av.av_length_head_update(h, acc, bk, k, step=3, **{n: t.clone() for n, t in init.items()})
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        out = av.av_length_head_update(h, acc, bk, k, step=3, want_grad_h=True, **st)
    for _ in range(3):
        for n, t in st.items():
            t.copy_(init[n])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in st:
            assert torch.equal(st[n], ref_state[n]), n
        for key in ("loss", "rate", "grad_h"):
            assert torch.equal(out[key], ref[key]), key
