"""Seeded synthetic inputs for paged-KV GQA attention.

This module only *builds inputs*: random BF16 tensors, page assignments, the
CSR block table and the position tensors.  It holds none of the attention
arithmetic, so both the CPU oracle (``oracle/``) and the HIP library's tests and
benchmark can draw the same bytes from it without sharing any of the method.

All randomness is numpy PCG64 from an explicit seed.  BF16 values are produced
by rounding float32 draws with torch's own float32 -> bfloat16 conversion and
stored as uint16 bit patterns.

Workload shapes (per-GPU head share; page size 16, head_dim 128, NHD layout):

* ``tiny_decode``      B=2, Hq=8, Hkv=2, 128 keys per row, 64-page pool.
* ``qwen3_8b_decode``  B=32, Hq=16, Hkv=4, lengths U{512..4096}, 16,384-page pool.
* ``invariance_row``   one 1,500-token row, Hq=32, Hkv=8 (alone, or row 3 of a batch of 8).
* ``chunked_prefill``  B=4 x 512-query chunks after prefixes 0/1024/2048/3584, Hq=32, Hkv=8.
* ``long_decode``      B in {1,2,4}, lengths 32K/64K/128K, Hq=32, Hkv=8, 40,960-page pool.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

PAGE_SIZE = 16
HEAD_DIM = 128
BF16_QNAN = np.uint16(0x7FC0)


def _to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_normal(rng: np.random.Generator, shape, chunk: int = 1 << 26) -> np.ndarray:
    """BF16 bit patterns of float32 N(0, 1) draws (drawn in chunks to bound host memory)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = _to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


@dataclass
class PagedBatch:
    """One paged-attention problem: tensors as numpy arrays (BF16 as uint16 bits)."""

    q: np.ndarray                   # uint16 [B, Hq, Sq, D]
    k_cache: np.ndarray             # uint16 [num_pages, PAGE_SIZE, Hkv, D]
    v_cache: np.ndarray             # uint16 [num_pages, PAGE_SIZE, Hkv, D]
    kv_indptr: np.ndarray           # int32 [B + 1]
    kv_indices: np.ndarray          # int32 [nnz]
    kv_last_page_len: np.ndarray    # int32 [B]
    cache_position: np.ndarray      # int32 [B, Sq]
    query_position_ids: np.ndarray  # int32 [B, Sq]
    key_position_ids: np.ndarray    # int32 [nnz * PAGE_SIZE]
    q_norm_weight: Optional[np.ndarray]  # float32 [D] or None
    k_norm_weight: Optional[np.ndarray]  # float32 [D] or None
    lengths: np.ndarray             # int64 [B]: logical KV length per row
    eps: float = 1e-6
    theta: float = 1e6
    rope_scale: float = 1.0
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_q_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def q_len(self) -> int:
        return int(self.q.shape[2])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_cache.shape[2])

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def nnz(self) -> int:
        return int(self.kv_indices.shape[0])

    def oracle_args(self):
        """Positional and keyword arguments in the order ``oracle.paged_attention`` takes them."""
        args = (self.q, self.k_cache, self.v_cache, self.kv_indptr, self.kv_indices,
                self.kv_last_page_len, self.query_position_ids, self.key_position_ids,
                self.q_norm_weight, self.k_norm_weight)
        kwargs = dict(eps=self.eps, theta=self.theta, scale=self.rope_scale)
        return args, kwargs


def csr_from_lengths(lengths: Sequence[int], page_order: np.ndarray):
    """CSR block table for rows of the given KV lengths.

    Row b takes ceil(L_b / 16) pages, consumed in order from ``page_order``.  A row
    with no keys has no pages and last_page_len 1 (the canonical inactive row).
    Returns (indptr, indices, last_page_len, key_position_ids).
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    pages = (lengths + PAGE_SIZE - 1) // PAGE_SIZE
    indptr = np.zeros(len(lengths) + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(pages)
    nnz = int(indptr[-1])
    if nnz > len(page_order):
        raise ValueError(f"pool too small: need {nnz} pages, have {len(page_order)}")
    indices = np.asarray(page_order[:nnz], dtype=np.int32)
    last = np.where(pages > 0, lengths - (pages - 1) * PAGE_SIZE, 1).astype(np.int32)
    key_pos = np.full(nnz * PAGE_SIZE, -1, dtype=np.int32)
    for b, L in enumerate(lengths):
        base = int(indptr[b]) * PAGE_SIZE
        key_pos[base:base + L] = np.arange(L, dtype=np.int32)
    return indptr, indices, last, key_pos


def make_batch(seed: int, lengths: Sequence[int], *, q_len: int, num_q_heads: int, num_kv_heads: int,
               num_pages: int, query_mode: str = "decode", canary: bool = True,
               page_order: Optional[np.ndarray] = None, norm: bool = True) -> PagedBatch:
    """Build a seeded batch.

    ``query_mode``: "decode" puts the q_len queries at positions L-q_len+1 .. L
    (for q_len 1, the single query sits at position L, after the cached keys);
    "prefill" puts them at L-q_len .. L-1 (the chunk's own keys are in the cache).
    ``canary``: pool pages no row uses are filled with BF16 NaN, so a stray read
    poisons the output instead of passing silently.
    ``page_order``: physical pages in the order rows consume them (default: a
    seeded permutation of the whole pool).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = np.asarray(lengths, dtype=np.int64)
    B = len(lengths)
    if page_order is None:
        page_order = rng.permutation(num_pages).astype(np.int32)
    indptr, indices, last, key_pos = csr_from_lengths(lengths, page_order)
    shape = (num_pages, PAGE_SIZE, num_kv_heads, HEAD_DIM)
    k_cache = bf16_normal(rng, shape)
    v_cache = bf16_normal(rng, shape)
    if canary:
        used = np.zeros(num_pages, dtype=bool)
        used[indices] = True
        k_cache[~used] = BF16_QNAN
        v_cache[~used] = BF16_QNAN
    q = bf16_normal(rng, (B, num_q_heads, q_len, HEAD_DIM))
    if norm:
        qw = rng.uniform(0.5, 1.5, HEAD_DIM).astype(np.float32)
        kw = rng.uniform(0.5, 1.5, HEAD_DIM).astype(np.float32)
    else:
        qw = kw = None
    if query_mode == "decode":
        first = lengths - q_len + 1
    elif query_mode == "prefill":
        first = lengths - q_len
    else:
        raise ValueError(query_mode)
    qpos = (first[:, None] + np.arange(q_len)[None, :]).astype(np.int32)
    return PagedBatch(q=q, k_cache=k_cache, v_cache=v_cache, kv_indptr=indptr, kv_indices=indices,
                      kv_last_page_len=last, cache_position=qpos.copy(), query_position_ids=qpos,
                      key_position_ids=key_pos, q_norm_weight=qw, k_norm_weight=kw, lengths=lengths,
                      meta=dict(seed=seed, query_mode=query_mode))


def permute_pages(batch: PagedBatch, seed: int) -> PagedBatch:
    """Same logical problem with every used page moved to a different physical page.

    The K/V contents follow their pages, so the logical K/V order, and hence the
    attention result, is unchanged.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(batch.num_pages)         # old page p -> new page perm[p]
    k = np.empty_like(batch.k_cache)
    v = np.empty_like(batch.v_cache)
    k[perm] = batch.k_cache
    v[perm] = batch.v_cache
    indices = perm[batch.kv_indices].astype(np.int32)
    return PagedBatch(**{**batch.__dict__, "k_cache": k, "v_cache": v, "kv_indices": indices,
                         "meta": {**batch.meta, "permuted": seed}})


# ----------------------------------------------------------------------------------------
# The named workloads.
# ----------------------------------------------------------------------------------------

def tiny_decode(seed: int = 1000, canary: bool = True) -> PagedBatch:
    """B=2, Hq=8, Hkv=2, 128 keys per row; each row's 8 pages drawn without replacement
    from a seeded shuffle of a 64-page pool (first 8 to row 0, next 8 to row 1)."""
    rng = np.random.Generator(np.random.PCG64(seed + 7))
    order = rng.permutation(64).astype(np.int32)
    return make_batch(seed, [128, 128], q_len=1, num_q_heads=8, num_kv_heads=2, num_pages=64,
                      page_order=order, canary=canary)


def qwen3_8b_decode_lengths(seed: int = 1001, batch: int = 32, lo: int = 512, hi: int = 4096) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed + 13))
    return rng.integers(lo, hi + 1, size=batch)


def qwen3_8b_decode(seed: int = 1001, canary: bool = True, num_pages: int = 16384) -> PagedBatch:
    """B=32, Hq=16, Hkv=4 (one GPU's share of Qwen3-8B at two-way head parallelism); kv lengths
    U{512..4096}; pages a seeded permutation of a 16,384-page pool; query at position L."""
    return make_batch(seed, qwen3_8b_decode_lengths(seed), q_len=1, num_q_heads=16, num_kv_heads=4,
                      num_pages=num_pages, canary=canary)


INVARIANCE_ROW_LEN = 1500
INVARIANCE_ROW_INDEX = 3


def invariance_batch(seed: int = 1002, alone: bool = True, canary: bool = True,
                     num_pages: int = 8192) -> PagedBatch:
    """The fixed 1,500-token row (Hq=32, Hkv=8), alone (B=1) or as row 3 of a batch of 8
    whose other rows have lengths U{64..8192}.

    The row's pages, K/V contents and query are the same bytes in both forms, so its
    result must be bitwise equal.
    """
    rng = np.random.Generator(np.random.PCG64(seed + 17))
    others = rng.integers(64, 8192 + 1, size=7)
    lengths = [int(x) for x in others[:INVARIANCE_ROW_INDEX]] + [INVARIANCE_ROW_LEN] + \
              [int(x) for x in others[INVARIANCE_ROW_INDEX:]]
    full = make_batch(seed, lengths, q_len=1, num_q_heads=32, num_kv_heads=8, num_pages=num_pages,
                      canary=canary)
    if not alone:
        return full
    b = INVARIANCE_ROW_INDEX
    lo, hi = int(full.kv_indptr[b]), int(full.kv_indptr[b + 1])
    indices = full.kv_indices[lo:hi].copy()
    kp = full.key_position_ids[lo * PAGE_SIZE:hi * PAGE_SIZE].copy()
    k, v = full.k_cache.copy(), full.v_cache.copy()
    if canary:
        used = np.zeros(num_pages, dtype=bool)
        used[indices] = True
        k[~used] = BF16_QNAN
        v[~used] = BF16_QNAN
    return PagedBatch(q=full.q[b:b + 1].copy(), k_cache=k, v_cache=v,
                      kv_indptr=np.array([0, hi - lo], dtype=np.int32), kv_indices=indices,
                      kv_last_page_len=full.kv_last_page_len[b:b + 1].copy(),
                      cache_position=full.cache_position[b:b + 1].copy(),
                      query_position_ids=full.query_position_ids[b:b + 1].copy(), key_position_ids=kp,
                      q_norm_weight=full.q_norm_weight, k_norm_weight=full.k_norm_weight,
                      lengths=full.lengths[b:b + 1].copy(), meta={**full.meta, "alone": True})


CHUNKED_PREFILL_PREFIXES = (0, 1024, 2048, 3584)


def chunked_prefill(seed: int = 1003, canary: bool = True, chunk: int = 512,
                    prefixes: Sequence[int] = CHUNKED_PREFILL_PREFIXES, num_q_heads: int = 32,
                    num_kv_heads: int = 8, num_pages: int = 4096) -> PagedBatch:
    """B=4 rows, each a 512-query chunk after a cached prefix of 0/1024/2048/3584 tokens.

    The cache holds prefix + chunk keys (pre-norm, pre-RoPE); query i of row b is at
    position prefix_b + i; causal visibility on logical positions."""
    lengths = [p + chunk for p in prefixes]
    return make_batch(seed, lengths, q_len=chunk, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                      num_pages=num_pages, query_mode="prefill", canary=canary)


LONG_DECODE_BATCHES = (1, 2, 4)
LONG_DECODE_LENGTHS = (32768, 65536, 131072)


def long_decode(batch: int, length: int, seed: int = 1004, canary: bool = False,
                num_pages: int = 40960) -> PagedBatch:
    """B rows of ``length`` keys each (Hq=32, Hkv=8), pages scattered over a 40,960-page pool."""
    return make_batch(seed, [length] * batch, q_len=1, num_q_heads=32, num_kv_heads=8,
                      num_pages=num_pages, canary=canary)
