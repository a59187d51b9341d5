"""Float64 CPU oracle for the AdaFlash verify + OPD pass.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py may import it.  The product path (the HIP library and its
Python binding) never imports, calls or links anything in this package, and
this package imports nothing from the product path.
"""

from .opd import (  # noqa: F401
    RowTerms,
    accepted_length,
    bf16_bits_to_f64,
    length_head,
    row_terms,
    target_argmax,
    verify_opd,
    clip_margin,
)
from .head_update import (  # noqa: F401
    ADAMW_DEFAULTS,
    adamw_step,
    head_loss_and_grads,
    length_head_update,
)
from .spec_sample import (  # noqa: F401
    accept_test,
    exponential_from_word,
    philox4x32_10,
    race_exponentials,
    race_uniforms,
    residual_keys,
    spec_verify,
)
from .lm_head import lm_head_backward  # noqa: F401
