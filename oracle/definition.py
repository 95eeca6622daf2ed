"""Plain CPU definition of deterministic paged-KV GQA attention (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.  It is slow on purpose: every step is the plain
definition written out with numpy, with no blocking, fusion or reordering.

Sources (web pages; cited by title and section):

* [RL-Kernel PR #279] "[WS2][PR7][Attention] Add FlashInfer RoPE-fused paged
  attention scaffold", section "Scope" (boundary table).
* [WS2 PR7] "WS2 PR7 Fused Attention Backend Alignment", sections "Original PR7
  Requirements", "Current Implementation", "FlashInfer RoPE Fusion",
  "Split-KV Policy", "Batch-Invariant Validation".
* [vllm-rlt PR #162] "flashinfer_fa2 backend for NVIDIA Ada (SM89)", sections
  "Summary", "Design notes", "Code audit" ("Data flows checked").
* [WS2 cross-config] "WS2 Attention Cross-Configuration Integration", section
  "H100 Attention input and projection boundary".

Numeric conventions (readings where the pages are silent; each is stated in
the function that applies it):

* Inputs q, k_cache, v_cache are BF16, handled here as their uint16 bit
  patterns so that no library conversion sits between the bytes and the math.
* The Q/K prologue (RMSNorm, then RoPE) is FP32 arithmetic with one IEEE
  round-to-nearest-even per operation and no fused multiply-add; the one
  reduction in it (the sum of squares) is exact.  Its result is rounded to
  BF16 (RNE) before attention: the "post-RoPE boundary" that both sides share.
* Scores, softmax, LSE and the output are computed in FP64, then rounded once
  (out to BF16 RNE, LSE to FP32 RNE).
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_bits_from_f32",
    "bf16_bits_from_f64",
    "bf16_round",
    "f32_from_bf16_bits",
    "row_lengths",
    "logical_kv",
    "rmsnorm_fp32",
    "rope_inv_freq",
    "rope_cos_sin",
    "rope_fp32",
    "prologue",
    "attention_fp64",
    "paged_attention",
]


# --------------------------------------------------------------------------------------
# BF16 encoding.  BF16 is the upper half of an IEEE binary32; conversion from
# binary32 is round-to-nearest, ties-to-even on the 16 discarded bits.
# --------------------------------------------------------------------------------------

def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Exact widening of BF16 bit patterns (uint16) to float32 values."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to BF16 (round to nearest, ties to even); returns uint16 bits.

    NaN maps to the canonical quiet NaN 0x7FC0; infinities and overflow behave as
    IEEE rounding prescribes (values past the largest BF16 round to infinity).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded = np.where(nan, np.uint16(0x7FC0), rounded)
    return rounded.astype(np.uint16)


def bf16_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """Round float64 values to BF16 (RNE) with a single rounding; returns uint16 bits.

    A plain float64 -> float32 -> BF16 chain rounds twice and can land on the
    wrong side of a BF16 midpoint.  When the float32 rounding was inexact and
    produced a value exactly halfway between two BF16 numbers, the float32 value
    is nudged one float32 ulp back toward the float64 value, after which the
    BF16 rounding is the correct single rounding of the float64 value.
    """
    x = np.asarray(x, dtype=np.float64)
    x32 = x.astype(np.float32)
    u = x32.view(np.uint32).copy()
    inexact = np.isfinite(x) & (x32.astype(np.float64) != x)
    on_mid = (u & np.uint32(0xFFFF)) == np.uint32(0x8000)
    fix = inexact & on_mid
    if fix.any():
        # moving the magnitude up or down by one ulp is +-1 on the bit pattern
        toward_zero = np.abs(x32.astype(np.float64)) > np.abs(x)
        step = np.where(toward_zero, np.uint32(0xFFFFFFFF), np.uint32(1))  # -1 or +1 (mod 2^32)
        u = np.where(fix, u + step, u)
    return bf16_bits_from_f32(u.view(np.float32))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest BF16 value (RNE), returned as float32."""
    return f32_from_bf16_bits(bf16_bits_from_f32(x))


# --------------------------------------------------------------------------------------
# Paged KV geometry.  [vllm-rlt PR #162] "Design notes" and "Code audit": the
# CSR block table is indptr (cumulative page counts), compact page indices and
# last_page_len; a row with no pages has last_page_len 1.  [RL-Kernel PR #279]
# "Scope": logical K/V and position order are materialised before arithmetic.
# --------------------------------------------------------------------------------------

def row_lengths(kv_indptr: np.ndarray, kv_last_page_len: np.ndarray, page_size: int) -> np.ndarray:
    """Logical KV length of each row: (pages - 1) * page_size + last_page_len, 0 for no pages."""
    indptr = np.asarray(kv_indptr, dtype=np.int64)
    last = np.asarray(kv_last_page_len, dtype=np.int64)
    pages = indptr[1:] - indptr[:-1]
    return np.where(pages > 0, (pages - 1) * page_size + last, 0)


def logical_kv(k_cache, v_cache, kv_indptr, kv_indices, kv_last_page_len, row: int, page_size: int):
    """Materialise row ``row``'s keys and values in logical order.

    Logical key j lives in physical page ``kv_indices[kv_indptr[row] + j // page_size]``
    at slot ``j % page_size``.  The caches are NHD: [num_pages, page_size, Hkv, D].
    Returns (K, V) as BF16 bit arrays [L, Hkv, D].
    """
    L = int(row_lengths(kv_indptr, kv_last_page_len, page_size)[row])
    j = np.arange(L, dtype=np.int64)
    pages = np.asarray(kv_indices, dtype=np.int64)[int(kv_indptr[row]) + j // page_size]
    slots = j % page_size
    return k_cache[pages, slots], v_cache[pages, slots]


# --------------------------------------------------------------------------------------
# Q/K prologue.  [RL-Kernel PR #279] "Scope": Q/K RMSNorm (Qwen3) and RoPE on
# both sides of the same post-RoPE boundary.  [WS2 cross-config] "H100 Attention
# input and projection boundary": the order inside the attention boundary is
# Q/K RMSNorm, then RoPE.  [WS2 PR7] "FlashInfer RoPE Fusion": Llama RoPE,
# theta 1e6, scale 1.0, rotary_dim = head_dim, rotate-half (non-interleaved),
# applied to pre-RoPE Q and the pre-RoPE K cache.
# --------------------------------------------------------------------------------------

def rmsnorm_fp32(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """Qwen3-style RMSNorm over the last axis (head_dim) in FP32.

    Reading (the pages fix neither the op order nor the reduction): with x the
    float32 values of the BF16 inputs and D = head_dim,

      ss   = sum_i x_i^2                      exact (each square of a BF16 value is exact in
                                              float32; their float64 sum is exact for any
                                              realistic exponent spread)
      ms   = RN32(ss / D)                     mean of squares, one rounding
      t    = RN32(ms + RN32(eps))             float32 add
      inv  = RN32(1 / sqrt(t))                correctly rounded reciprocal square root,
                                              evaluated as float64 sqrt and divide
      y_i  = RN32(RN32(x_i * inv) * w_i)      two float32 multiplies, left to right
    """
    x = np.asarray(x, dtype=np.float32)
    w = np.asarray(weight, dtype=np.float32)
    d = x.shape[-1]
    ss = np.sum(np.square(x.astype(np.float64)), axis=-1)
    ms = (ss / d).astype(np.float32)
    t = ms + np.float32(eps)
    inv = (1.0 / np.sqrt(t.astype(np.float64))).astype(np.float32)
    return (x * inv[..., None]) * w


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """Llama inverse frequencies theta^(-2i/D), i < D/2, in float64 (libm pow)."""
    return np.array([math.pow(theta, -(2.0 * i) / head_dim) for i in range(head_dim // 2)],
                    dtype=np.float64)


def rope_cos_sin(positions: np.ndarray, head_dim: int, theta: float, scale: float):
    """cos/sin of the exact RoPE angles, rounded to float32.

    Reading: the angle (pos / scale) * theta^(-2i/D) is formed in float64 and
    cos/sin are evaluated in float64, then rounded once to float32.  (A float32
    product pos * inv_freq is off by ~1e-3 rad at position 1.3e5, which the pages'
    accuracy gates would notice, so the exact angle is the reading taken.)
    Returns (cos, sin), each [..., D/2] float32.
    """
    pos = np.asarray(positions, dtype=np.float64) / float(scale)
    ang = pos[..., None] * rope_inv_freq(head_dim, theta)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rope_fp32(y: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE in float32 without fused multiply-add.

    For i < D/2 the pair (i, i + D/2) rotates by the angle of frequency i:
      out_i       = RN32(RN32(y_i * c_i)       - RN32(y_{i+D/2} * s_i))
      out_{i+D/2} = RN32(RN32(y_{i+D/2} * c_i) + RN32(y_i * s_i))
    """
    y = np.asarray(y, dtype=np.float32)
    h = y.shape[-1] // 2
    y1, y2 = y[..., :h], y[..., h:]
    return np.concatenate([y1 * cos - y2 * sin, y2 * cos + y1 * sin], axis=-1)


def prologue(x_bits: np.ndarray, weight, positions, eps: float, theta: float, scale: float) -> np.ndarray:
    """bf16(RoPE(RMSNorm(x) * w, pos)) for BF16 inputs x [..., D]; returns float32 values on the BF16 grid.

    ``weight=None`` skips the RMSNorm (a cache that already holds normalised K).
    ``positions`` broadcasts against x.shape[:-1].
    """
    x = f32_from_bf16_bits(x_bits)
    y = x if weight is None else rmsnorm_fp32(x, weight, eps)
    c, s = rope_cos_sin(positions, x.shape[-1], theta, scale)
    return bf16_round(rope_fp32(y, c, s))


# --------------------------------------------------------------------------------------
# Attention.  [RL-Kernel PR #279] "Scope": FP32 attention-domain LSE, GQA packing
# fixed by the head layout, no auto split.  [WS2 PR7] "Original PR7 Requirements":
# LSE shaped [B, Hq, Sq]; causal visibility on logical positions ("Current
# Implementation": cache_position == query_position_ids, trailing positions).
# The oracle computes in float64, so it has no reduction order to fix.
# --------------------------------------------------------------------------------------

def attention_fp64(qhat: np.ndarray, khat: np.ndarray, v: np.ndarray,
                   q_pos: np.ndarray, k_pos: np.ndarray, sm_scale: float):
    """Causal softmax attention of one query head group against one KV head.

    qhat [G, Sq, D], khat [L, D], v [L, D] (float64 values); q_pos [Sq], k_pos [L].
    Key j is visible to query i iff k_pos[j] <= q_pos[i].
      s_ij  = (qhat_i . khat_j) * sm_scale
      lse_i = log(sum_{j visible} exp(s_ij))     (natural log; -inf if nothing is visible)
      out_i = sum_{j visible} exp(s_ij - lse_i) v_j (0 if nothing is visible)
    Returns (out [G, Sq, D], lse [G, Sq]) in float64.
    """
    qhat = np.asarray(qhat, dtype=np.float64)
    G, Sq, D = qhat.shape
    L = khat.shape[0]
    if L == 0:
        return np.zeros((G, Sq, D)), np.full((G, Sq), -np.inf)
    s = np.matmul(qhat, np.asarray(khat, dtype=np.float64).T) * sm_scale        # [G, Sq, L]
    visible = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]           # [Sq, L]
    s = np.where(visible[None], s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    any_visible = np.isfinite(m)
    m_safe = np.where(any_visible, m, 0.0)
    e = np.exp(s - m_safe)
    total = np.sum(e, axis=-1, keepdims=True)
    with np.errstate(divide="ignore"):
        lse = np.where(any_visible, m_safe + np.log(total), -np.inf)
    p = np.where(any_visible, np.exp(s - np.where(any_visible, lse, 0.0)), 0.0)
    out = np.matmul(p, np.asarray(v, dtype=np.float64))
    return out, lse[..., 0]


def paged_attention(q, k_cache, v_cache, kv_indptr, kv_indices, kv_last_page_len,
                    query_position_ids, key_position_ids, q_norm_weight, k_norm_weight,
                    *, eps: float = 1e-6, theta: float = 1e6, scale: float = 1.0,
                    rows=None, q_heads=None):
    """Reference result of paged GQA attention for the selected rows and query heads.

    q: BF16 bits [B, Hq, Sq, D] (pre-norm, pre-RoPE); k_cache, v_cache: BF16 bits
    [num_pages, page_size, Hkv, D] (NHD; K pre-norm, pre-RoPE).  kv_indptr [B+1],
    kv_indices [nnz], kv_last_page_len [B]: the CSR block table.
    query_position_ids [B, Sq]; key_position_ids [nnz * page_size], where logical
    key j of row b sits at offset kv_indptr[b] * page_size + j.
    q_norm_weight / k_norm_weight: float32 [D] or None (no RMSNorm on that side).

    Query head h reads KV head h // (Hq / Hkv) (contiguous GQA groups).  The
    softmax scale is 1/sqrt(D).  Rows share nothing, so every row is computed on
    its own.

    Returns (out_bits uint16 [R, H, Sq, D], lse float32 [R, H, Sq]) for the
    selected rows R (default all) and query heads H (default all), in the order
    given.
    """
    B, Hq, Sq, D = q.shape
    page_size, Hkv = k_cache.shape[1], k_cache.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    rows = list(range(B)) if rows is None else list(rows)
    q_heads = list(range(Hq)) if q_heads is None else list(q_heads)
    sm_scale = 1.0 / math.sqrt(D)
    out_bits = np.zeros((len(rows), len(q_heads), Sq, D), dtype=np.uint16)
    lse = np.zeros((len(rows), len(q_heads), Sq), dtype=np.float32)
    lengths = row_lengths(kv_indptr, kv_last_page_len, page_size)
    for ri, b in enumerate(rows):
        L = int(lengths[b])
        kb, vb = logical_kv(k_cache, v_cache, kv_indptr, kv_indices, kv_last_page_len, b, page_size)
        base = int(kv_indptr[b]) * page_size
        k_pos = np.asarray(key_position_ids[base:base + L], dtype=np.int64)
        q_pos = np.asarray(query_position_ids[b], dtype=np.int64)
        for hkv in sorted({h // group for h in q_heads}):
            heads = [(hi, h) for hi, h in enumerate(q_heads) if h // group == hkv]
            khat = prologue(kb[:, hkv], k_norm_weight, k_pos, eps, theta, scale)
            v = f32_from_bf16_bits(vb[:, hkv])
            qhat = np.stack([prologue(q[b, h], q_norm_weight, q_pos, eps, theta, scale) for _, h in heads])
            o, l = attention_fp64(qhat, khat, v, q_pos, k_pos, sm_scale)
            for gi, (hi, _) in enumerate(heads):
                out_bits[ri, hi] = bf16_bits_from_f64(o[gi])
                lse[ri, hi] = l[gi].astype(np.float32)
    return out_bits, lse
