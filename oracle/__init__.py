"""CPU oracle for absorbed MLA decode — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never does.
"""
from .mla_oracle import (  # noqa: F401
    D_KVC, D_LATENT, D_ROPE, LSE_ATOL, OUT_ATOL, OUT_RTOL,
    absorb_query, as_f64, attend_one, bf16_bits_to_f64, brute_force_decode,
    explicit_mla_decode, gather_request_rows, merge_partials, oracle_decode,
    parity_report, split_partials,
)
