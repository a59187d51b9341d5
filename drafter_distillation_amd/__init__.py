"""AdaFlash verify + on-policy-distillation pass for AMD Instinct MI355X.

The work is done by the gfx950 HIP library libav.so (C ABI: include/av.h);
this package only binds it.  Build with `python -m drafter_distillation_amd.build`.
"""

from ._lib import (  # noqa: F401
    AV_BF16,
    AV_DEV_BAD_OFFSETS,
    AV_DEV_TIMEOUT,
    AV_EHIP,
    AV_EINVAL,
    AV_EUNSUPPORTED,
    AV_F32,
    AV_MAX_K,
    AV_OK,
    AV_ROUND_CEIL,
    AV_ROUND_FLOOR,
    AVError,
    LIB_PATH,
    av_head_update_workspace_bytes,
    av_length_head,
    av_length_head_update,
    av_lm_head_bwd,
    av_spec_verify,
    av_spec_workspace_bytes,
    av_status_str,
    av_verify_opd_bwd,
    av_verify_opd_fwd,
    av_workspace_bytes,
    lib,
    workspace,
)
