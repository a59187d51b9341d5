"""The gfx950 code of the library is free of the two code-generation hazards
that drafter_distillation_amd.isa_check looks for (wide-store data registers
rewritten too early, lane loops around scalar operands).  Compiles the kernels
to assembly with the build flags (hipcc cross-compiles; no GPU needed)."""

import os
import shutil

import pytest

from drafter_distillation_amd import build as B
from drafter_distillation_amd import isa_check as C


@pytest.fixture(scope="module", params=["av_kernels.hip", "av_lmhead.hip"])
def asm(request):
    if not os.path.exists(B._hipcc()) and shutil.which(B._hipcc()) is None:
        pytest.skip("hipcc not available")
    return C.compile_asm(os.path.join(B.CSRC, request.param))


def test_no_wide_store_or_lane_loop_hazards(asm):
    probs = C.check(asm)
    assert not probs, "\n".join(probs[:20])


def test_checker_flags_a_planted_hazard():
    bad = "\n".join([
        "_Zplanted:",
        "\tbuffer_store_dwordx4 v[4:7], v12, s[48:51], s6 offen",
        "\tv_add_u32_e32 v4, 0x400, v12",
        "\ts_endpgm",
        ".Lfunc_end0:",
    ])
    good = bad.replace("\tv_add_u32_e32", "\ts_nop 1\n\tv_add_u32_e32")
    assert len(C.check(bad)) == 1
    assert C.check(good) == []


def test_checker_flags_a_lane_loop():
    loop = "\n".join([
        "_Zplanted:",
        ".LBB0_1:",
        "\tv_readfirstlane_b32 s15, v5",
        "\tv_cmp_eq_u32_e32 vcc, s15, v5",
        "\ts_and_saveexec_b64 vcc, vcc",
        "\tbuffer_store_dwordx4 v[62:65], v74, s[48:51], s15 offen",
        "\ts_nop 1",
        "\ts_endpgm",
        ".Lfunc_end0:",
    ])
    assert any("lane loop" in p for p in C.check(loop))


def test_checker_follows_branches():
    """The window after a wide store is followed into both successors of a
    conditional branch: a write at the branch target one wait state after the
    branch is flagged, two are not."""
    def prog(target_pad):
        return "\n".join([
            "_Zplanted:",
            "\tscratch_store_dwordx4 off, v[4:7], off offset:16",
            "\ts_cbranch_execz .LBB0_2",
            "\ts_nop 1",
            "\tv_mov_b32_e32 v4, 0",
            ".LBB0_2:",
            *target_pad,
            "\tv_mov_b32_e32 v5, 0",
            "\ts_endpgm",
            ".Lfunc_end0:",
        ])
    assert len(C.check(prog([]))) == 1
    assert C.check(prog(["\ts_or_b64 exec, exec, s[2:3]"])) == []
