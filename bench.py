#!/usr/bin/env python3
"""Benchmark of the AdaFlash verify + OPD hot path on one MI355X.

One step = one pass of the whole path over the concurrent workload
(B=128 requests, k=16 draft positions, V=151936, bf16 logits):
  av_length_head   (pooled state -> b_k per request)
  av_verify_opd_fwd (target argmax, acceptance scan, clipped reverse-KL + CE
                    loss, per-request and total loss, fp32 gradient w.r.t. the
                    drafter logits), one fused kernel launch.
Inputs are generated on the host (seeded), copied to HBM before timing, and
stay resident.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

`--workload head_update` measures instead the online update of the length
head (av_length_head_update) on the same workload's head: B=128 pooled
states of H=4096, labels from one verification pass, gradients with respect
to w, bias and h, one AdamW step per call.

`--workload spec` measures sampling-based verification (av_spec_verify) of
the same workload: acceptance tests with the caller's uniforms on every
verified row, and the residual draw at each request's first rejection.

`--workload lm_head` measures the backward of the drafter's LM head
(av_lm_head_bwd) on the same workload's bfloat16 gradient: d hid = dz W and
d W = dz^T hid with R=2048, V=151936, H=4096 (two bf16 GEMMs).

`--workload tiny` and `--workload single` report the latency of one step
(length head + fused pass) on one request: B=1, k=16, V=4096 float32 logits
(H=256), and B=1, k=16, V=151936 bfloat16 logits (H=4096).

`--workload ragged` and `--workload long` time the fused pass on the ragged
workload (B=128, only the b_k verified rows of each request stored) and on
the long one (B=64, k=32, V=262144); `--workload long_sweep` prints one line
per (lambda, tau) in {0, 0.5, 1} x {0.05, 0.1, 1e9} on the long workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused verify+OPD fwd/bwd GB/s and % HBM peak at B=128,k=16,V=151936 bf16"
HBM_PEAK_GBS = 8000.0
KERNEL_SRC_DIR = os.path.join(ROOT, "drafter_distillation_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_concurrent_traffic.json")


# Sources of the fused kernel and its launch (the LM-head GEMMs are not part of it).
FUSED_SOURCES = ("av_api.hip", "av_internal.h", "av_kernels.hip")


def kernel_sha() -> str:
    """Hash of the fused kernel's and its launch's sources: counter readings
    are stale once it changes."""
    hsh = hashlib.sha256()
    for name in FUSED_SOURCES:
        with open(os.path.join(KERNEL_SRC_DIR, name), "rb") as f:
            hsh.update(name.encode() + b"\0" + f.read())
    return hsh.hexdigest()[:16]


def algorithmic_bytes(B, k, V, H, R, Rv, elem=2, gelem=4, lse1=False):
    """Bytes the pass must move at least once (per step).

    fused kernel: zp of every stored row (target argmax is defined for all),
    zq of verified rows, the fp32 gradient of every stored row (zeros for
    unverified rows are part of the output), draft tokens, b_k, and the small
    per-row / per-request outputs (with a reverse-KL temperature also the
    plain log-sum-exp of zq per row).  length head: h, w, rate and b_k.
    """
    fused = (elem * V * R + elem * V * Rv + gelem * V * R
             + 4 * R + 4 * B            # draft, bk
             + 4 * R + 4 * R + 16 * R   # argmax, row loss, row stats
             + (4 * R if lse1 else 0)   # lse of zq at temperature 1
             + 4 * B + 4 * B + 4)       # acc, req loss, total
    head = 4 * B * H + 4 * H + 8 * B
    return fused, head


def measured_traffic():
    """HBM bytes per fused launch from the committed rocprofv3 counter runs,
    or None when they were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != kernel_sha():
        return None
    return t.get("bytes_per_launch")


FUSED_KERNEL_PREFIX = "void avk::(anonymous namespace)::fused_kernel<"
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _counter_rows(csv_path: str, counter: str):
    import csv

    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") == counter:
                yield row["Kernel_Name"], int(row["Grid_Size"]), float(row["Counter_Value"])


def summarize_traffic(fetch_csv: str, write_csv: str, copy_mib: int) -> dict:
    """HBM bytes per fused launch from two rocprofv3 --pmc runs (FETCH_SIZE,
    WRITE_SIZE; KiB per dispatch) of `bench.py --copy-calibration-mib N`.

    Each counter is scaled by known bytes / counter bytes of the plain
    device-to-device copy of N MiB that run performs (the copy reads N MiB and
    writes N MiB).  Only the largest copy dispatches (the calibration copy)
    are used for the factor.
    """
    known = copy_mib * 1024.0  # KiB read (and written) by the calibration copy
    out = {"kernel_sha": kernel_sha(), "copy_calibration_mib": copy_mib}
    total = 0.0
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = list(_counter_rows(path, name))
        fused = [v for k, g, v in rows if k.startswith(FUSED_KERNEL_PREFIX)]
        copies = [(g, v) for k, g, v in rows if k == COPY_KERNEL]
        if not fused or not copies:
            raise SystemExit(f"{path}: no {name} rows for the fused kernel or the copy")
        gmax = max(g for g, _ in copies)
        cal = [v for g, v in copies if g == gmax]
        cal_kib = sum(cal) / len(cal)
        factor = known / cal_kib
        fused_kib = sum(fused) / len(fused)
        out[name] = {"fused_kib_per_dispatch": round(fused_kib, 3), "dispatches": len(fused),
                     "copy_kib_per_dispatch": round(cal_kib, 3), "copy_dispatches": len(cal),
                     "factor": round(factor, 6)}
        total += fused_kib * 1024.0 * factor
    out["bytes_per_launch"] = int(round(total))
    return out


def copy_calibration(torch, dev, mib: int, reps: int = 3) -> None:
    """A plain device-to-device copy of `mib` MiB, run `reps` times outside the
    timed region, as the known-size reference for the HBM byte counters."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


# Host cores the oracle baseline may use: the affinity mask, at most 16 (one
# GPU's share of a GPU host's CPUs).
MAX_ORACLE_CORES = 16

# The workload the forked oracle workers read (set before the pool starts).
_ORACLE_JOB: dict = {}


def _oracle_request(b: int) -> float:
    """Worker: the float64 oracle on request b of _ORACLE_JOB's workload
    (decode, length head of that request, the pass); returns its seconds."""
    import numpy as np

    import oracle
    from threadpoolctl import threadpool_limits

    j = _ORACLE_JOB
    w, k = j["w"], j["w"].k

    def decode(a):
        return oracle.bf16_bits_to_f64(a) if w.dtype == "bf16" else a.astype(np.float64)

    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        if w.row_off is not None:  # ragged: the request's verified rows only, no length head
            r0, r1 = int(w.row_off[b]), int(w.row_off[b + 1])
            oracle.verify_opd(decode(w.zp[r0:r1]), decode(w.zq[r0:r1]), w.draft[r0:r1], k=k, lam=w.lam,
                              tau=w.tau, grad_scale=1.0, row_off=np.array([0, r1 - r0]),
                              temperature=j["temperature"])
        else:
            rows = slice(b * k, (b + 1) * k)
            zp, zq = decode(w.zp[rows]), decode(w.zq[rows])
            oracle.length_head(w.h[b:b + 1], w.w, w.bias, w.gamma, k)
            oracle.verify_opd(zp, zq, w.draft[rows], k=k, lam=w.lam, tau=w.tau, grad_scale=1.0,
                              bk=j["bk"][b:b + 1], temperature=j["temperature"])
        return time.perf_counter() - t0


def cpu_baseline(w, single_requests: int = 16, temperature: float = 1.0):
    """The float64 oracle, untuned, on the same workload: all B requests
    spread over the host's cores (a fork pool over requests, one numpy thread
    each), and the first `single_requests` requests on one core.  Reported in
    the same unit as the GPU line (algorithmic GB/s).  Run before the process
    touches the GPU, so the forked workers start from a process without a
    device context."""
    import multiprocessing as mp

    import numpy as np

    import oracle

    if w.row_off is None:
        _, bk, _ = oracle.length_head(w.h, w.w, w.bias, w.gamma, w.k)
    else:
        bk = np.diff(w.row_off)
    cores = max(1, min(MAX_ORACLE_CORES, len(os.sched_getaffinity(0))))
    _ORACLE_JOB.update(w=w, bk=bk, temperature=temperature)
    try:
        t0 = time.perf_counter()
        with mp.get_context("fork").Pool(cores) as pool:
            busy = sum(pool.map(_oracle_request, range(w.B), chunksize=1))
        dt = time.perf_counter() - t0
        t1 = time.perf_counter()
        for b in range(single_requests):
            _oracle_request(b)
        dt1 = time.perf_counter() - t1
    finally:
        _ORACLE_JOB.clear()
    Rv = int(np.clip(bk, 1, w.k).sum())
    ragged = w.row_off is not None
    H = 0 if ragged else w.H  # the ragged workload runs no length head
    fused, head = algorithmic_bytes(w.B, w.k, w.V, H, w.R, Rv, lse1=temperature != 1.0)
    bk1 = np.clip(bk[:single_requests], 1, w.k)
    r1 = int(bk1.sum()) if ragged else single_requests * w.k
    f1, h1 = algorithmic_bytes(single_requests, w.k, w.V, H, r1, int(bk1.sum()), lse1=temperature != 1.0)
    return {
        "value": round((fused + head) / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"all {w.B} requests of the same workload ({w.R} rows, {Rv} verified), float64 numpy, "
                  f"{cores} worker processes over requests (one numpy thread each), {dt:.1f} s wall, "
                  f"{busy:.1f} s of CPU work; single core: first {single_requests} requests, {dt1:.1f} s",
        "seconds": round(dt, 3),
        "cpu_seconds": round(busy, 3),
        "single_core_value": round((f1 + h1) / dt1 / 1e9, 4),
    }


def head_update_bytes(B, H):
    """Bytes the head update must move at least once: h, acc and b_k read;
    w and its two moments read and written; the bias and its moments; the
    gradient with respect to h, the rates and the loss written."""
    return 4 * B * H + 8 * B + 3 * 2 * 4 * H + 3 * 2 * 4 + 4 * B * H + 4 * B + 4


def cpu_baseline_head_update(h, w, bias, acc, bk, k, reps: int):
    """The float64 oracle's update, single-threaded, `reps` consecutive steps."""
    import oracle
    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        state, ww, bb = None, w, bias
        for _ in range(reps):
            r = oracle.length_head_update(h, ww, bb, acc, bk, k, state)
            ww, bb, state = r["w"], r["bias"], r["state"]
        dt = (time.perf_counter() - t0) / reps
    return {
        "value": round(dt * 1e6, 1),
        "unit": "us per update",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{reps} consecutive updates of the same head (B={h.shape[0]}, H={h.shape[1]}), "
                  f"float64 numpy, one thread",
        "seconds": round(dt * reps, 3),
    }


def bench_head_update(args):
    import numpy as np
    import torch

    import drafter_distillation_amd as dd
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dd.lib()
    w = synth.make("concurrent", seed=args.seed)
    B, k, V, H = w.B, w.k, w.V, w.H
    h = torch.from_numpy(w.h).to(dev)
    wt = torch.from_numpy(w.w).to(dev)
    bk = torch.empty(B, dtype=torch.int32, device=dev)
    dd.av_length_head(h, wt, w.bias, w.gamma, k, bk_out=bk)
    # labels from one verification pass over the same workload
    zp = torch.from_numpy(w.zp.view(np.int16)).view(torch.bfloat16).to(dev)
    zq = torch.from_numpy(w.zq.view(np.int16)).view(torch.bfloat16).to(dev)
    out = dd.av_verify_opd_fwd(zp, zq, torch.from_numpy(w.draft).to(dev), k=k, bk=bk, lam=w.lam,
                               tau=w.tau, want_grad=False)
    acc = out["acc_len"]
    torch.cuda.synchronize()
    del zp, zq, out
    state = dict(w=wt.clone(), bias=torch.tensor([w.bias], dtype=torch.float32, device=dev),
                 m_w=torch.zeros(H, dtype=torch.float32, device=dev),
                 v_w=torch.zeros(H, dtype=torch.float32, device=dev),
                 m_b=torch.zeros(1, dtype=torch.float32, device=dev),
                 v_b=torch.zeros(1, dtype=torch.float32, device=dev))
    # The host takes longer to issue an update than the GPU takes to run it,
    # so the timed region replays a captured graph of `steps` consecutive
    # updates (their step numbers are fixed at capture; the work is the same).
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    n = 0

    def update():
        nonlocal n
        n += 1
        dd.av_length_head_update(h, acc, bk, k, step=n, want_grad_h=True, **state)

    with torch.cuda.stream(cap):
        for _ in range(args.warmup):
            update()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for _ in range(args.steps):
            update()
    torch.cuda.synchronize()
    with torch.cuda.stream(cap):
        graph.replay()  # warm replay
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(cap)
        graph.replay()
        e1.record(cap)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern_us = e0.elapsed_time(e1) * 1e3 / args.steps
    nbytes = head_update_bytes(B, H)
    achieved = nbytes / (kern_us * 1e-6) / 1e9
    line = {
        "metric": "length-head online update (MSE vs acc/b_k, grads w.r.t. w, bias, h, AdamW step) "
                  "us per update at B=128, H=4096",
        "value": round(kern_us, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {
            "workload": "head update: the concurrent workload's length head (B=128, H=4096, k=16), "
                        "labels from one verification pass, float32 parameters and moments",
            "B": B, "H": H, "k": k, "seed": args.seed, "bytes_per_update": nbytes,
            "launches_per_update": 2, "timing": "HIP events around one replay of a captured "
                                                 "graph of `steps` consecutive updates",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_head_update(
            w.h.astype(np.float64), w.w.astype(np.float64), float(w.bias),
            acc.cpu().numpy(), bk.cpu().numpy(), k, reps=20)
    print(json.dumps(line), flush=True)


def spec_bytes(V, Rv, n_rej, elem=2, stats_given=False):
    """Bytes sampling verification must move at least once: zp and zq of every
    verified row (its statistics), zp and zq of each request's rejected row
    again for the residual draw (the statistics are needed first), the
    uniforms, drafts and per-row records, and the per-request outputs.  With
    the row statistics given (the fused pass's first sweep computed them):
    the two gathered logits, the two statistics, the draft and the uniform of
    each verified row, and zp and zq of each rejected row once."""
    if stats_given:
        return (2 * elem + 8 + 8) * Rv + 2 * elem * V * n_rej + 8 * n_rej
    return 2 * elem * V * Rv + 2 * elem * V * n_rej + 12 * Rv + 8 * n_rej


def bench_spec(args):
    import numpy as np
    import torch

    import drafter_distillation_amd as dd
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dd.lib()
    w = synth.make("concurrent", seed=args.seed)
    B, k, V, H, R = w.B, w.k, w.V, w.H, w.R
    zp = torch.from_numpy(w.zp.view(np.int16)).view(torch.bfloat16).to(dev)
    zq = torch.from_numpy(w.zq.view(np.int16)).view(torch.bfloat16).to(dev)
    draft = torch.from_numpy(w.draft).to(dev)
    bk = torch.empty(B, dtype=torch.int32, device=dev)
    dd.av_length_head(torch.from_numpy(w.h).to(dev), torch.from_numpy(w.w).to(dev), w.bias, w.gamma, k,
                      bk_out=bk)
    u = torch.from_numpy(np.random.default_rng(args.seed + 1).random(R).astype(np.float32)).to(dev)
    seed = 0x5EED0000 + args.seed
    out = None
    stream = torch.cuda.current_stream(dev)
    stats_in = None
    if args.spec_stats == "fused":  # the row statistics of a fused pass on the same inputs
        stats_in = dd.av_verify_opd_fwd(zp, zq, draft, k=k, bk=bk, lam=w.lam, tau=w.tau,
                                        want_grad=False)["row_stats"]
        torch.cuda.synchronize()

    def step(ev0=None, ev1=None):
        nonlocal out
        if ev0 is not None:
            ev0.record(stream)
        out = dd.av_spec_verify(zp, zq, draft, u, k=k, seed=seed, bk=bk, out=out, stats_in=stats_in)
        if ev1 is not None:
            ev1.record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        step(e0, e1)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / len(evs)
    bkh = torch.clamp(bk, 1, k).cpu().numpy()
    acc = out["acc_len"].cpu().numpy()
    Rv, n_rej = int(bkh.sum()), int((acc < bkh).sum())
    nbytes = spec_bytes(V, Rv, n_rej, stats_given=stats_in is not None)
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    line = {
        "metric": "sampling-based block verification GB/s at B=128,k=16,V=151936 bf16"
                  + (", row statistics from the fused pass" if stats_in is not None else ""),
        "value": round(achieved, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "spec: the concurrent workload (B=128, k=16, V=151936, bf16 logits, greedy "
                        "drafts of the drafter logits, b_k from the length head), uniforms seeded",
            "B": B, "k": k, "V": V, "verified_rows": Rv, "rejecting_requests": n_rej,
            "accepted_positions": int(acc.sum()), "bytes_per_step": nbytes,
            "kernel_ms": round(kern_ms, 4), "launches_per_step": 3,
            "row_statistics": "given (fused pass)" if stats_in is not None else "computed",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
        },
    }
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_limits
        nb = 16
        uh = u.cpu().numpy()
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            zpd = oracle.bf16_bits_to_f64(w.zp[:nb * k])
            zqd = oracle.bf16_bits_to_f64(w.zq[:nb * k])
            res = oracle.spec_verify(zpd, zqd, w.draft[:nb * k], uh[:nb * k], k=k, seed=seed, bk=bkh[:nb])
            dt = time.perf_counter() - t0
        sb = spec_bytes(V, int(bkh[:nb].sum()), int((res["acc"] < bkh[:nb]).sum()))
        line["cpu_baseline"] = {
            "value": round(sb / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {nb} of {B} requests of the same workload, float64 numpy, one thread, "
                      f"{dt:.1f} s", "seconds": round(dt, 3)}
    print(json.dumps(line), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_lm_head(args):
    import numpy as np
    import torch

    import drafter_distillation_amd as dd
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dd.lib()
    w = synth.make("concurrent", seed=args.seed)
    B, k, V, R = w.B, w.k, w.V, w.R
    H = 4096
    zp = torch.from_numpy(w.zp.view(np.int16)).view(torch.bfloat16).to(dev)
    zq = torch.from_numpy(w.zq.view(np.int16)).view(torch.bfloat16).to(dev)
    bk = torch.empty(B, dtype=torch.int32, device=dev)
    dd.av_length_head(torch.from_numpy(w.h).to(dev), torch.from_numpy(w.w).to(dev), w.bias, w.gamma, k,
                      bk_out=bk)
    dz = dd.av_verify_opd_fwd(zp, zq, torch.from_numpy(w.draft).to(dev), k=k, bk=bk, lam=w.lam, tau=w.tau,
                              grad_scale=1.0 / float(torch.clamp(bk, 1, k).sum()),
                              grad_dtype=torch.bfloat16)["grad"]
    del zp, zq
    g = torch.Generator(device=dev).manual_seed(args.seed)
    wl = (torch.randn((V, H), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    hid = torch.randn((R, H), generator=g, device=dev).to(torch.bfloat16)
    stream = torch.cuda.current_stream(dev)

    def timed(fn, steps):
        """Average of per-call HIP event pairs on the launching stream (ms),
        and the wall time of the loop (s)."""
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        t0 = time.perf_counter()
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return sum(e0.elapsed_time(e1) for e0, e1 in evs) / steps, time.perf_counter() - t0

    kern_ms, elapsed = timed(lambda: dd.av_lm_head_bwd(dz, wl, hid), args.steps)
    hid_ms, _ = timed(lambda: dd.av_lm_head_bwd(dz, wl, None, want_d_w=False), args.steps)
    w_ms, _ = timed(lambda: dd.av_lm_head_bwd(dz, None, hid, want_d_hid=False), args.steps)
    # the same two products through torch.mm (bfloat16 outputs, rocBLAS /
    # hipBLASLt), for context; the transposed dz is made before timing
    dzt = dz.t().contiguous()
    torch_hid_ms, _ = timed(lambda: torch.mm(dz, wl), args.steps)
    torch_w_ms, _ = timed(lambda: torch.mm(dzt, hid), args.steps)
    del dzt
    flops1 = 2.0 * R * V * H
    flops = 2 * flops1
    tflops = flops / (kern_ms * 1e-3) / 1e12

    def tf(ms):
        return round(flops1 / (ms * 1e-3) / 1e12, 1)

    line = {
        "metric": "drafter LM-head backward (d hid = dz W, d W = dz^T hid) TFLOP/s at R=2048, V=151936, "
                  "H=4096 bf16",
        "value": round(tflops, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "lm_head: dz = the concurrent workload's bf16 gradient (R=2048, V=151936), "
                        "W [V, 4096] and hid [2048, 4096] random bf16, float32 accumulation and outputs",
            "R": R, "V": V, "H": H, "flop_per_step": flops, "kernel_ms": round(kern_ms, 4),
            "gemms": "gemm_kernel (own v_mfma_f32_32x32x16_bf16 tiles)",
            "d_hid_ms": round(hid_ms, 4), "d_hid_tflops": tf(hid_ms),
            "d_w_ms": round(w_ms, 4), "d_w_tflops": tf(w_ms),
            "torch_mm_bf16_out": {"d_hid_ms": round(torch_hid_ms, 4), "d_hid_tflops": tf(torch_hid_ms),
                                  "d_w_ms": round(torch_w_ms, 4), "d_w_tflops": tf(torch_w_ms)},
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None,
        },
    }
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_limits
        rows = 2
        dzh = dz[:rows].float().cpu().numpy().astype(np.float64)
        wh = wl.float().cpu().numpy().astype(np.float64)
        hh = hid[:rows].float().cpu().numpy().astype(np.float64)
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            oracle.lm_head_backward(dzh, wh, hh)
            dt = time.perf_counter() - t0
        sflops = 2 * 2.0 * rows * V * H
        line["cpu_baseline"] = {
            "value": round(sflops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} of {R} rows (both products), float64 numpy, one thread, {dt:.1f} s",
            "seconds": round(dt, 3)}
    print(json.dumps(line), flush=True)


def bench_bwd(args):
    """The standalone backward (av_verify_opd_bwd) on the concurrent workload:
    the gradient from the statistics a forward call without gradient saved.
    Bytes per call: zp and zq of the verified rows read once, the gradient of
    every row written (zeros for unverified rows), the row statistics and
    argmax of the verified rows read."""
    import numpy as np
    import torch

    import drafter_distillation_amd as dd
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dd.lib()
    w = synth.make("concurrent", seed=args.seed)
    B, k, V, R = w.B, w.k, w.V, w.R
    zp = torch.from_numpy(w.zp.view(np.int16)).view(torch.bfloat16).to(dev)
    zq = torch.from_numpy(w.zq.view(np.int16)).view(torch.bfloat16).to(dev)
    draft = torch.from_numpy(w.draft).to(dev)
    bk = torch.empty(B, dtype=torch.int32, device=dev)
    dd.av_length_head(torch.from_numpy(w.h).to(dev), torch.from_numpy(w.w).to(dev), w.bias, w.gamma, k,
                      bk_out=bk)
    fwd = dd.av_verify_opd_fwd(zp, zq, draft, k=k, bk=bk, lam=w.lam, tau=w.tau, want_grad=False)
    gdt = torch.bfloat16 if args.grad == "bf16" else torch.float32
    grad = torch.empty((R, V), dtype=gdt, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev0=None, ev1=None):
        if ev0 is not None:
            ev0.record(stream)
        dd.av_verify_opd_bwd(zp, zq, fwd["tgt_argmax"], fwd["row_stats"], k=k, bk=bk, lam=w.lam,
                             tau=w.tau, grad_scale=1.0, grad=grad, grad_dtype=gdt)
        if ev1 is not None:
            ev1.record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    Rv = int(torch.clamp(bk, 1, k).sum().item())
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        step(e0, e1)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gelem = 2 if args.grad == "bf16" else 4
    nbytes = 2 * 2 * V * Rv + gelem * V * R + (16 + 4) * Rv + 4 * B
    kern_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / len(evs)
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    line = {
        "metric": "standalone OPD backward GB/s at B=128,k=16,V=151936 bf16"
                  + (", bf16 gradient" if args.grad == "bf16" else ""),
        "value": round(achieved, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "bwd: the concurrent workload (B=128, k=16, V=151936, bf16 logits, b_k from the "
                        "length head); gradient from the saved row statistics",
            "B": B, "k": k, "V": V, "rows": R, "verified_rows": Rv, "grad": args.grad,
            "bytes_per_call": nbytes, "kernel_ms": round(kern_ms, 4),
        },
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
    }
    print(json.dumps(line))


def bench_fused_other(args):
    """The fused pass on the ragged workload (B=128, k=16, V=151936, only the
    b_k verified rows of each request stored) or the long one (B=64, k=32,
    V=262144, b_k from the length head, H=5120), kernel only, timed as the
    default bench; `long_sweep` prints one line per (lambda, tau) of the long
    workload's grid on the same resident inputs."""
    import numpy as np
    import torch

    import drafter_distillation_amd as dd
    import synth

    name = "long" if args.workload == "long_sweep" else args.workload
    w = synth.make(name, seed=args.seed)
    # the oracle baseline runs first, in worker processes forked before this
    # process touches the GPU
    cpu_line = None if args.no_cpu_baseline else cpu_baseline(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dd.lib()
    B, k, V, R = w.B, w.k, w.V, w.R
    zp = torch.from_numpy(w.zp.view(np.int16)).view(torch.bfloat16).to(dev)
    zq = torch.from_numpy(w.zq.view(np.int16)).view(torch.bfloat16).to(dev)
    draft = torch.from_numpy(w.draft).to(dev)
    kw = {}
    if w.row_off is not None:
        kw["row_off"] = torch.from_numpy(w.row_off).to(dev)
        bkh = np.diff(w.row_off)
        Rv = R
    else:
        bk = torch.empty(B, dtype=torch.int32, device=dev)
        dd.av_length_head(torch.from_numpy(w.h).to(dev), torch.from_numpy(w.w).to(dev), w.bias, w.gamma, k,
                          bk_out=bk)
        kw["bk"] = bk
        bkh = np.clip(bk.cpu().numpy(), 1, k)
        Rv = int(bkh.sum())
    gdt = torch.bfloat16 if args.grad == "bf16" else torch.float32
    gelem = 2 if args.grad == "bf16" else 4
    fused_b, _ = algorithmic_bytes(B, k, V, 0, R, Rv, gelem=gelem)
    stream = torch.cuda.current_stream(dev)
    pairs = [(lam, tau) for lam in (0.0, 0.5, 1.0) for tau in (0.05, 0.1, 1e9)] \
        if args.workload == "long_sweep" else [(w.lam, w.tau)]
    out = None
    for lam, tau in pairs:
        def step(ev0=None, ev1=None):
            nonlocal out
            if ev0 is not None:
                ev0.record(stream)
            out = dd.av_verify_opd_fwd(zp, zq, draft, k=k, lam=lam, tau=tau, grad_scale=1.0, out=out,
                                       grad_dtype=gdt, **kw)
            if ev1 is not None:
                ev1.record(stream)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        if int(out["status"].item()) != 0:
            raise RuntimeError(f"device status {int(out['status'].item())}")
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        t0 = time.perf_counter()
        for e0, e1 in evs:
            step(e0, e1)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        kern_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / len(evs)
        achieved = fused_b / (kern_ms * 1e-3) / 1e9
        acch = out["acc_len"].cpu().numpy()
        desc = {"ragged": f"ragged: B={B} requests, k={k}, V={V}, bf16 logits, only the {R} verified rows stored "
                          "(b_k drawn with p proportional to 1/b)",
                "long": f"long: B={B} requests, k={k}, V={V}, bf16 logits, b_k from the length head (H={w.H})"}
        line = {
            "metric": f"fused verify+OPD fwd/bwd GB/s, {name} workload",
            "value": round(achieved, 2),
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(elapsed / args.steps * 1e3, 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "f32",
            "data": "synthetic",
            "config": {"workload": desc[name] + f", lambda={lam}, tau={tau:g}, {args.grad} gradient",
                       "B": B, "k": k, "V": V, "rows": R, "verified_rows": Rv, "lambda": lam, "tau": tau,
                       "bytes_per_call": fused_b, "kernel_ms": round(kern_ms, 4),
                       "rows_per_s": round(R / (kern_ms * 1e-3), 1),
                       "bk_hist_1_to_k": np.bincount(bkh, minlength=k + 1)[1:].tolist(),
                       "accepted_hist_0_to_k": np.bincount(acch, minlength=k + 1).tolist()},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
        }
        if cpu_line is not None and (lam, tau) == (w.lam, w.tau):
            line["cpu_baseline"] = cpu_line
        print(json.dumps(line), flush=True)


def bench_latency(args):
    """One step (length head + fused pass with gradient) on one request: the
    tiny workload (B=1, k=16, V=4096 float32 logits, H=256) or the single one
    (B=1, k=16, V=151936 bfloat16, H=4096).  Both are latency-bound, so the
    line reports microseconds per step (HIP events around each step), with the
    float64 oracle's time for the same step on one core beside it."""
    import numpy as np

    import oracle
    import synth

    w = synth.make(args.workload, seed=args.seed)
    B, k, V, H, R = w.B, w.k, w.V, w.H, w.R
    _, bk_ref, _ = oracle.length_head(w.h, w.w, w.bias, w.gamma, k)
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        reps = 5
        t0 = time.perf_counter()
        for _ in range(reps):
            zpd = oracle.bf16_bits_to_f64(w.zp) if w.dtype == "bf16" else w.zp.astype(np.float64)
            zqd = oracle.bf16_bits_to_f64(w.zq) if w.dtype == "bf16" else w.zq.astype(np.float64)
            oracle.length_head(w.h, w.w, w.bias, w.gamma, k)
            oracle.verify_opd(zpd, zqd, w.draft, k=k, lam=w.lam, tau=w.tau, grad_scale=1.0, bk=bk_ref)
        cpu_us = (time.perf_counter() - t0) / reps * 1e6

    import torch

    import drafter_distillation_amd as dd

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dd.lib()
    if w.dtype == "bf16":
        zp = torch.from_numpy(w.zp.view(np.int16)).view(torch.bfloat16).to(dev)
        zq = torch.from_numpy(w.zq.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        zp = torch.from_numpy(w.zp).to(dev)
        zq = torch.from_numpy(w.zq).to(dev)
    draft = torch.from_numpy(w.draft).to(dev)
    h = torch.from_numpy(w.h).to(dev)
    wt = torch.from_numpy(w.w).to(dev)
    rate = torch.empty(B, dtype=torch.float32, device=dev)
    bk = torch.empty(B, dtype=torch.int32, device=dev)
    out = None
    stream = torch.cuda.current_stream(dev)

    def step():
        nonlocal out
        dd.av_length_head(h, wt, w.bias, w.gamma, k, rate_out=rate, bk_out=bk)
        out = dd.av_verify_opd_fwd(zp, zq, draft, k=k, bk=bk, lam=w.lam, tau=w.tau, grad_scale=1.0, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(out["status"].item()) != 0:
        raise RuntimeError(f"device status {int(out['status'].item())}")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
    us_med = us[len(us) // 2]
    Rv = int(np.clip(bk.cpu().numpy(), 1, k).sum())
    elem = 2 if w.dtype == "bf16" else 4
    fused_b, head_b = algorithmic_bytes(B, k, V, H, R, Rv, elem=elem)
    line = {
        "metric": f"fused verify+OPD step latency (length head + fused pass) us at B=1,k={k},V={V} {w.dtype}",
        "value": round(us_med, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: B=1 request, k={k}, V={V}, {w.dtype} logits, b_k from the "
                               f"length head (H={H}), lambda={w.lam}, tau={w.tau}",
                   "B": B, "k": k, "V": V, "H": H, "verified_rows": Rv, "bytes_per_step": fused_b + head_b,
                   "us_min": round(us[0], 2), "us_p90": round(us[int(0.9 * (len(us) - 1))], 2),
                   "timing": "HIP events around each step (two launches), median"},
        "roofline": {"bound": "hbm", "achieved": round((fused_b + head_b) / (us_med * 1e-6) / 1e9, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round((fused_b + head_b) / (us_med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None, "note": "latency-bound: a handful of rows for 256 CUs"},
        "cpu_baseline": {"value": round(cpu_us, 1), "unit": "us", "cores": 1, "kind": "oracle",
                         "sample": f"the same step, float64 numpy, one thread, mean of {reps}"},
    }
    print(json.dumps(line), flush=True)


def bench_hbm_probe(args):
    """What the memory system delivers for the fused pass's byte patterns
    without its arithmetic (drafter_distillation_amd/probe/hbm_probe.hip, run
    as a child process): the achievable rates that the fused kernel's
    algorithmic bandwidth is compared with, next to the 8 TB/s peak."""
    import subprocess

    from drafter_distillation_amd.build import PROBE_BIN

    if not os.path.exists(PROBE_BIN):
        raise SystemExit(f"{PROBE_BIN} is missing: build it with `python -m drafter_distillation_amd.build`")
    out = subprocess.run([PROBE_BIN], capture_output=True, text=True, check=True).stdout
    runs = []
    for line in out.splitlines():
        pat, block, per_cu, us, gbs = line.split()
        runs.append({"pattern": pat, "block": int(block), "workgroups_per_cu": int(per_cu),
                     "us": float(us), "GBs": float(gbs)})
    best = {}
    for r in runs:
        if r["pattern"] not in best or r["GBs"] > best[r["pattern"]]["GBs"]:
            best[r["pattern"]] = r
    rows1024 = max((r for r in runs if r["pattern"] == "rows" and r["block"] == 1024), key=lambda r: r["GBs"])
    line = {
        "metric": "HBM bandwidth of the fused pass's byte patterns without arithmetic (GB/s)",
        "value": rows1024["GBs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "higher_is_better": True,
        "data": "synthetic",
        "config": {
            "workload": "2048 rows of V=151936 bf16 zp and zq (622 MB each), a 1245 MB float32 gradient; "
                        "value: one 1024-thread workgroup per row reads the row, barrier, writes its "
                        "gradient (a verified row's phases)",
            "best_by_pattern_GBs": {k: v["GBs"] for k, v in best.items()},
            "frac_of_8TBs_by_pattern": {k: round(v["GBs"] / HBM_PEAK_GBS, 4) for k, v in best.items()},
            "runs": runs,
        },
    }
    print(json.dumps(line))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--grad", choices=["f32", "bf16"], default="f32",
                    help="gradient output type of the fused pass (default float32)")
    ap.add_argument("--spec-stats", choices=["own", "fused"], default="own",
                    help="spec workload: compute the row statistics (own) or take the fused pass's")
    ap.add_argument("--temperature", type=float, default=1.0,
                    help="reverse-KL temperature of the fused pass (default 1: the plain pass)")
    ap.add_argument("--workload", choices=["concurrent", "tiny", "single", "ragged", "long", "long_sweep",
                                            "head_update", "spec", "lm_head", "hbm_probe", "bwd"],
                    default="concurrent",
                    help="concurrent: the fused verify+OPD step (default); head_update: the "
                         "length head's online update; spec: sampling-based verification")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run a plain copy of this many MiB before warmup (counter calibration)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic file from two rocprofv3 --pmc counter CSVs and exit")
    args = ap.parse_args()

    if args.summarize_traffic:
        t = summarize_traffic(*args.summarize_traffic, args.copy_calibration_mib or 1024)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(t, f, indent=1)
            f.write("\n")
        print(json.dumps(t))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build's path runs on a single MI355X "
              "(the multi-GPU split over requests is described in DESIGN.md); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    if args.workload == "head_update":
        bench_head_update(args)
        return
    if args.workload == "spec":
        bench_spec(args)
        return
    if args.workload == "lm_head":
        bench_lm_head(args)
        return
    if args.workload == "hbm_probe":
        bench_hbm_probe(args)
        return
    if args.workload == "bwd":
        bench_bwd(args)
        return
    if args.workload in ("ragged", "long", "long_sweep"):
        bench_fused_other(args)
        return
    if args.workload in ("tiny", "single"):
        bench_latency(args)
        return

    import numpy as np

    import synth

    w = synth.make("concurrent", seed=args.seed)
    # the oracle baseline runs first, in worker processes forked before this
    # process touches the GPU
    cpu_line = None if args.no_cpu_baseline else cpu_baseline(w, temperature=args.temperature)

    import torch

    import drafter_distillation_amd as dd

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dd.lib()

    if args.copy_calibration_mib > 0:
        copy_calibration(torch, dev, args.copy_calibration_mib)

    zp = torch.from_numpy(w.zp.view(np.int16)).view(torch.bfloat16).to(dev)
    zq = torch.from_numpy(w.zq.view(np.int16)).view(torch.bfloat16).to(dev)
    draft = torch.from_numpy(w.draft).to(dev)
    h = torch.from_numpy(w.h).to(dev)
    wt = torch.from_numpy(w.w).to(dev)
    B, k, V, H, R = w.B, w.k, w.V, w.H, w.R
    rate = torch.empty(B, dtype=torch.float32, device=dev)
    bk = torch.empty(B, dtype=torch.int32, device=dev)
    out = {
        "tgt_argmax": torch.empty(R, dtype=torch.int32, device=dev),
        "acc_len": torch.empty(B, dtype=torch.int32, device=dev),
        "row_loss": torch.empty(R, dtype=torch.float32, device=dev),
        "req_loss": torch.empty(B, dtype=torch.float32, device=dev),
        "total_loss": torch.empty(1, dtype=torch.float32, device=dev),
        "row_stats": torch.empty((R, 4), dtype=torch.float32, device=dev),
        "grad": torch.empty((R, V), dtype=torch.bfloat16 if args.grad == "bf16" else torch.float32,
                            device=dev),
        "status": torch.empty(1, dtype=torch.int32, device=dev),
    }
    tempered = args.temperature != 1.0
    if tempered:
        out["lse_q1"] = torch.empty(R, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev0=None, ev1=None):
        dd.av_length_head(h, wt, w.bias, w.gamma, k, rate_out=rate, bk_out=bk)
        if ev0 is not None:
            ev0.record(stream)
        dd.av_verify_opd_fwd(zp, zq, draft, k=k, bk=bk, lam=w.lam, tau=w.tau,
                             grad_scale=1.0, out=out, grad_dtype=out["grad"].dtype,
                             temperature=args.temperature, want_lse_q1=tempered)
        if ev1 is not None:
            ev1.record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(out["status"].item()) != 0:
        raise RuntimeError(f"device status {int(out['status'].item())}")
    Rv = int(torch.clamp(bk, 1, k).sum().item())

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        step(e0, e1)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if int(out["status"].item()) != 0:
        raise RuntimeError(f"device status {int(out['status'].item())}")

    gelem = 2 if args.grad == "bf16" else 4
    fused_b, head_b = algorithmic_bytes(B, k, V, H, R, Rv, gelem=gelem, lse1=tempered)
    ms_step = elapsed / args.steps * 1e3
    bkh = np.clip(bk.cpu().numpy(), 1, k)
    acch = out["acc_len"].cpu().numpy()
    value = (fused_b + head_b) * args.steps / elapsed / 1e9
    kern_ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    kern_avg_ms = sum(kern_ms) / len(kern_ms)
    achieved = fused_b / (kern_avg_ms * 1e-3) / 1e9
    unverified_grad = gelem * V * (R - Rv)

    metric = METRIC if args.grad == "f32" else METRIC + ", bf16 gradient"
    if tempered:
        metric += f", reverse-KL temperature {args.temperature:g}"
    line = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"concurrent: B=128 requests, k=16, V=151936, bf16 logits, {args.grad} gradient, "
                        "b_k from the length head (H=4096), lambda=0.5, tau=0.1"
                        + (f", reverse-KL temperature {args.temperature:g}" if tempered else ""),
            "B": B, "k": k, "V": V, "H": H, "rows": R, "verified_rows": Rv,
            "logits": "bf16", "grad": args.grad, "seed": args.seed, "temperature": args.temperature,
            "rows_per_s": round(R / (ms_step * 1e-3), 1),
            "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
            "bytes_per_step": fused_b + head_b,
            "value_without_zero_fill_GBs": round((fused_b + head_b - unverified_grad) * args.steps
                                                 / elapsed / 1e9, 2),
            "kernel_ms": round(kern_avg_ms, 4),
            "bk_hist_1_to_k": np.bincount(bkh, minlength=k + 1)[1:].tolist(),
            "accepted_hist_0_to_k": np.bincount(acch, minlength=k + 1).tolist(),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic() if args.grad == "f32" and not tempered else None,
        },
    }
    if cpu_line is not None:
        line["cpu_baseline"] = cpu_line
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
