"""Seeded synthetic inputs for the verify + OPD pass (shared by the tests, the
bench and the oracle checks; holds none of the method's arithmetic)."""

from .gen import (  # noqa: F401
    CONFIGS,
    Workload,
    bf16_bits_to_float,
    make,
    request_rows,
    to_bf16_bits,
)
