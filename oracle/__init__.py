"""CPU float64 oracle for absorbed MLA decode and the MLA query front end.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the GPU library.
"""
from .codecs import (  # noqa: F401
    E4M3_TABLE,
    bf16_bits_to_f64,
    bf16_round,
    e4m3_round,
    e4m3_to_f64,
    f64_to_bf16_bits,
    f64_to_e4m3,
)
from .mla_oracle import (  # noqa: F401
    attend,
    combine,
    dequant_rows,
    mla_decode,
    mla_query,
    physical_rows,
    valid_positions,
)
