"""Seeded synthetic inputs for the MLA latent-cache workloads.

This package only draws random numbers, rounds them to the storage format and
lays them out (pages, page tables, poison fills).  It holds none of the
attention arithmetic: the fp64 oracle (``oracle/``) and the HIP library
(``mla_latent_kv_31_amd``) both consume what it produces, and neither shares
any other code with the other.
"""

from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits,
    bf16_from_bits,
    bf16_round,
    make_decode_inputs,
    make_prefill_inputs,
    make_toy_inputs,
    paginate,
)
