"""CPU oracle for deterministic paged-KV grouped-query attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything under ``oracle/``; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library: no kernels, headers, helpers, tables or constants.

What it computes, and the passages it follows, are documented function by
function in :mod:`oracle.definition` (attention), :mod:`oracle.csr` (the CSR
block table built from a dense one) and :mod:`oracle.backward` (the gradients of
full-prefill attention).  Every function there is pinned by
``tests/test_oracle_pins.py`` against closed forms, invariants, library
routines or brute force on tiny inputs; none is "parity unpinned".
"""

from .definition import (  # noqa: F401
    bf16_bits_from_f32,
    bf16_bits_from_f64,
    bf16_round,
    f32_from_bf16_bits,
    row_lengths,
    logical_kv,
    rmsnorm_fp32,
    rope_inv_freq,
    rope_cos_sin,
    rope_fp32,
    prologue,
    attention_fp64,
    paged_attention,
)
from .csr import csr_from_block_table  # noqa: F401
from .backward import prefill_forward_backward  # noqa: F401
