"""Plain fp64 CPU oracle for the groupwise low-bit dequantize + matrix multiply.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The library
(``w4_groupwise_gemm_amd``) never imports it and shares no code with it: the
oracle reads the canonical weight format directly and never the repacked
device layout.

Every function here is pinned by ``tests/test_oracle_pins.py`` against things
fixed outside the oracle (exact rational brute force, literal byte fixtures,
closed forms, integer matmul special cases, and the invariants the pages
state).  See ``oracle.reference`` for the definitions and their sources.
"""
from .reference import (  # noqa: F401
    unpack_codes,
    dequantize,
    linear,
    linear_rows,
    silu,
    swiglu,
    linear_add,
    fp16_round,
    bf16_value,
    quantize_a8,
    linear_a8,
    rel_l2,
)
