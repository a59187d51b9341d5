"""Static check of the gfx950 code of the library for two code-generation
hazards the compiler does not guard against on this target:

* wide-store data: a store of more than 8 bytes (buffer/global/flat/scratch
  dwordx3/x4) keeps reading its data registers after it issues; any VALU
  write to one of them must come at least two wait states later, on every
  path through the branches that follow (a function's end within that
  window also counts as a problem);
* lane loops: a wave-uniform scalar operand that the compiler could not prove
  uniform makes it loop over lanes (readfirstlane / compare / saveexec around
  the instruction), which is slow and has clobbered store data.

Usage: python -m drafter_distillation_amd.isa_check [file.s]
(without a file, compiles the library's kernel sources to assembly with the
build flags).
"""

from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

WIDE_STORE = re.compile(r"^(buffer|global|flat|scratch)_store_dwordx[34]\b")
MIN_WAIT_STATES = 2


def _regs(tok: str) -> set:
    tok = tok.rstrip(",")
    m = re.match(r"^v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"^v(\d+)$", tok)
    if m:
        return {int(m.group(1))}
    return set()


def _store_data(ins: str) -> set:
    ops = ins.split(None, 1)[1].split(",")
    ops = [o.strip() for o in ops]
    if ins.startswith("buffer_store"):
        return _regs(ops[0])
    # global/flat/scratch: vaddr (or off), vdata, ...
    return _regs(ops[1])


def _valu_dst(ins: str) -> set:
    if not ins.startswith("v_") or ins.startswith(("v_cmp", "v_readlane", "v_readfirstlane")):
        return set()
    parts = ins.split(None, 1)
    if len(parts) < 2:
        return set()
    return _regs(parts[1].split(",")[0].strip())


def _wait_states(ins: str) -> int:
    m = re.match(r"^s_nop\s+(\d+)", ins)
    return int(m.group(1)) + 1 if m else 1


def functions(asm: str):
    """Yield (name, [instruction lines]) for each function in an asm file."""
    name, body = None, []
    for raw in asm.split("\n"):
        line = raw.split(";")[0].rstrip()
        m = re.match(r"^(_Z\S+):\s*$", line)
        if m:
            if name:
                yield name, body
            name, body = m.group(1), []
            continue
        if name is None:
            continue
        if line.strip().startswith(".Lfunc_end"):
            yield name, body
            name, body = None, []
            continue
        s = line.strip()
        if not s or s.startswith(".") and not s.endswith(":"):
            continue
        body.append(s)


def _follow(body: list, labels: dict, start: int, data: set, waited: int, seen: set):
    """Walks every path from body[start] until MIN_WAIT_STATES have passed;
    returns the first instruction on a path that writes `data` too early (or
    leaves the function), else None."""
    i = start
    while i < len(body) and waited < MIN_WAIT_STATES:
        if (i, waited) in seen:
            return None
        seen.add((i, waited))
        nxt = body[i]
        if nxt.endswith(":"):
            i += 1
            continue
        if nxt.startswith(("s_setpc", "s_endpgm")):
            return nxt
        if nxt.startswith(("s_branch", "s_cbranch")):
            tgt = nxt.split()[-1]
            if tgt not in labels:
                return nxt
            hit = _follow(body, labels, labels[tgt], data, waited + 1, seen)
            if hit or nxt.startswith("s_branch"):
                return hit
            waited += 1
            i += 1
            continue
        if _valu_dst(nxt) & data:
            return nxt
        waited += _wait_states(nxt)
        i += 1
    return None


def check(asm: str) -> list:
    problems = []
    for fn, body in functions(asm):
        labels = {ins[:-1]: j for j, ins in enumerate(body) if ins.endswith(":")}
        for i, ins in enumerate(body):
            if WIDE_STORE.match(ins):
                hit = _follow(body, labels, i + 1, _store_data(ins), 0, set())
                if hit:
                    problems.append(f"{fn}: '{ins}' data may be overwritten by '{hit}' within "
                                    f"{MIN_WAIT_STATES} wait states")
            if ins.startswith("v_readfirstlane_b32"):
                sreg = ins.split()[1].rstrip(",")
                window = body[i + 1:i + 5]
                if any(w.startswith("v_cmp_eq") and sreg in w for w in window) and \
                        any("saveexec" in w for w in window):
                    problems.append(f"{fn}: lane loop at '{ins}'")
    return problems


def compile_asm(src: str, extra=()) -> str:
    from . import build as B

    with tempfile.TemporaryDirectory() as td:
        out = os.path.join(td, "k.s")
        flags = [*B.HIPCC_FLAGS, *B.SOURCE_FLAGS.get(os.path.basename(src), []), *extra]
        subprocess.check_call([B._hipcc(), *flags, "--cuda-device-only", "-S", src, "-o", out],
                              stderr=subprocess.DEVNULL)
        with open(out) as f:
            return f.read()


def main(argv=None) -> int:
    argv = sys.argv[1:] if argv is None else argv
    if argv:
        with open(argv[0]) as f:
            asm = f.read()
    else:
        from . import build as B

        asm = "\n".join(compile_asm(os.path.join(B.CSRC, f)) for f in ("av_kernels.hip", "av_lmhead.hip"))
    probs = check(asm)
    for p in probs:
        print(p)
    print(f"{len(probs)} problem(s)")
    return 1 if probs else 0


if __name__ == "__main__":
    sys.exit(main())
