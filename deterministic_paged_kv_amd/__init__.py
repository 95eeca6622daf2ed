"""Deterministic, batch-invariant paged-KV GQA attention for AMD MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
``include/pa.h`` (``libpa.so``, built in-tree by ``build.py``).  This package is
the thin Python binding over it: :class:`Plan`, :func:`validate_metadata`,
:func:`decode`, :func:`prefill`, the full-prefill backward :func:`prefill_backward`,
and the device-side CSR builder :func:`build_csr` with its plan-width helper
:func:`width_bucket`.  Importing it does not load the
library; the first call does, and raises if it is not built.
"""

from .binding import (  # noqa: F401
    PA_SPLIT_DISABLED,
    PA_SPLIT_FIXED,
    PagedAttentionError,
    Plan,
    build_csr,
    decode,
    decode_no_alloc,
    decode_workspace,
    decode_workspace_size,
    load,
    prefill,
    prefill_backward,
    prefill_backward_workspace_size,
    prefill_workspace_size,
    status_string,
    validate_metadata,
    width_bucket,
)
