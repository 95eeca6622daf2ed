"""Plain CPU construction of the CSR block table from a dense one (TEST INFRASTRUCTURE ONLY).

Only ``tests/`` may import this module (like the rest of ``oracle/``).  It shares no
code with the HIP library.

Source: [vllm-rlt PR #162] "flashinfer_fa2 backend for NVIDIA Ada (SM89)", sections
"Design notes" (the metadata is indptr, compact indices and last_page_len, built once
per traversal from the block table and the context lengths) and "Code audit" ("Data
flows checked": indptr is the running sum of ceil(len / 16), the compact indices are
the rows' live table entries packed back to back, rows with no keys report
last_page_len 1; the audit's finding that the construction was only checked without an
empty row).

Readings where the pages are silent (the same ones the library states in include/pa.h):

* the output indices array keeps the fixed shape B * width; slots past the compact
  count hold -1;
* a length outside [0, 16 * width] has no representation: the row takes its whole table
  row and last_page_len 0 (an invalid value, so validation and the attention kernels
  flag the row instead of silently truncating it).
"""

from __future__ import annotations

import numpy as np

PAGE = 16


def csr_from_block_table(block_table, lens):
    """(indptr [B+1], indices [B*W], last_page_len [B]) as int32 arrays, one row at a time."""
    table = np.asarray(block_table, dtype=np.int64)
    lens = [int(x) for x in np.asarray(lens).reshape(-1)]
    B = len(lens)
    W = int(table.shape[1]) if table.ndim == 2 else 0
    indptr = [0]
    indices = []
    last = []
    for b in range(B):
        L = lens[b]
        if 0 <= L <= PAGE * W:
            pages = -(-L // PAGE)                      # ceil(L / 16)
            last.append(1 if L == 0 else L - (pages - 1) * PAGE)
        else:
            pages = W
            last.append(0)
        for j in range(pages):
            indices.append(int(table[b, j]))
        indptr.append(indptr[-1] + pages)
    indices += [-1] * (B * W - len(indices))
    return (np.array(indptr, dtype=np.int32), np.array(indices, dtype=np.int32),
            np.array(last, dtype=np.int32))
