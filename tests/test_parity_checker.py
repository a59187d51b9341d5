"""The GPU parity checker itself, on the CPU: fed outputs made by the oracle
(in float32, as the GPU returns them) it reports nothing; fed the same
outputs with one planted error it reports that error, whether the rows are
checked in this process or in forked worker processes."""

import numpy as np

import oracle
import synth
from parity_util import check_workload, decode_rows


def oracle_outputs(w, bk, lam, tau, gs):
    zp, zq = decode_rows(w, "zp", slice(None)), decode_rows(w, "zq", slice(None))
    ref = oracle.verify_opd(zp, zq, w.draft, k=w.k, lam=lam, tau=tau, grad_scale=gs, bk=bk)
    return {"tgt_argmax": ref["tgt_argmax"].astype(np.int32), "acc_len": ref["acc_len"].astype(np.int32),
            "row_loss": ref["row_loss"].astype(np.float32), "req_loss": ref["req_loss"].astype(np.float32),
            "total_loss": np.array([ref["total_loss"]], np.float32),
            "row_stats": ref["row_stats"].astype(np.float32), "grad": ref["grad"].astype(np.float32),
            "status": np.zeros(1, np.int32)}


def test_checker_serial_and_forked_agree():
    w = synth.make("concurrent", B=4, V=3000)
    bk = np.array([16, 3, 9, 1])
    out = oracle_outputs(w, bk, 0.5, 0.1, 0.25)
    assert check_workload(out, w, bk, 0.5, 0.1, 0.25) == []
    assert check_workload(out, w, bk, 0.5, 0.1, 0.25, workers=2) == []
    bad = {k: v.copy() for k, v in out.items()}
    bad["grad"][18, 77] += 0.01 + 0.1 * abs(bad["grad"][18, 77])  # a wrong gradient entry
    bad["grad"][20, 5] = 1e-3                                     # unverified row must stay zero
    for workers in (0, 2):
        errs = check_workload(bad, w, bk, 0.5, 0.1, 0.25, workers=workers)
        assert any(e.startswith("row 18: ") and "grad" in e for e in errs), errs
        assert any(e.startswith("row 20: ") for e in errs), errs
