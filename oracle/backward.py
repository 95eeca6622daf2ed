"""Plain CPU gradients of full-prefill attention (TEST INFRASTRUCTURE ONLY).

Only ``tests/`` and ``bench.py``'s ``cpu_baseline`` leg may import this module.  It shares
no code with the HIP library.

Sources: [RL-Kernel PR #279] "[WS2][PR7][Attention] Add FlashInfer RoPE-fused paged
attention scaffold", section "Scope" (the backward of the strict attention path must be
deterministic, dropout 0); [WS2 PR7] "WS2 PR7 Fused Attention Backend Alignment", sections
"Goal" (a training full-prefill lane beside the rollout paged lane) and "Original PR7
Requirements" (the training forward is full prefill / teacher forcing; dq/dk/dv belong to
the training backward); the forward it differentiates is the one in :mod:`oracle.definition`
(Q/K RMSNorm, then rotate-half RoPE, then causal softmax attention with GQA).

Readings where the pages are silent:

* "Full prefill" is the training layout: dense q [B, Hq, S, D], k and v [B, Hkv, S, D]; the
  keys of row b are its own S tokens; token i of row b sits at positions[b, i] for both
  its query and its key; key j is visible to query i iff positions[b, j] <= positions[b, i].
* The forward is the forward reference's: q^ and k^ are its post-RoPE BF16 values, and the
  attention runs in float64 on them.  The gradients pass through the BF16 roundings of q^,
  k^ (the post-RoPE boundary) and of out unchanged (straight-through); every step is
  differentiated in float64.  dout is the gradient of out.
* Gradients are returned for the pre-norm inputs q, k, v and for the two RMSNorm weights
  (shared by all heads and tokens).
"""

from __future__ import annotations

import math

import numpy as np

from .definition import f32_from_bf16_bits, prologue, rope_cos_sin


def _norm_rope_forward(x, w, cos, sin, eps):
    """Exact-arithmetic prologue: y = x r w (r = (mean x^2 + eps)^-1/2), then rotate-half RoPE.
    Without a weight (w None) there is no RMSNorm, as in the forward reference: y = x.
    x [..., D] float64.  Returns (rotated, r)."""
    d = x.shape[-1]
    r = 1.0 / np.sqrt(np.sum(x * x, axis=-1) / d + eps)
    y = x if w is None else x * r[..., None] * w
    h = d // 2
    y1, y2 = y[..., :h], y[..., h:]
    return np.concatenate([y1 * cos - y2 * sin, y2 * cos + y1 * sin], axis=-1), r


def _norm_rope_backward(x, w, cos, sin, r, g):
    """Gradient of the prologue: g is d loss / d rotated [..., D].  Returns (dx, dw or None).

    RoPE is a rotation, so its backward is the inverse rotation:
      dy1 = g1 c + g2 s,  dy2 = -g1 s + g2 c.
    RMSNorm y = x r w with r = (sum(x^2)/D + eps)^-1/2:
      dx_j = r w_j dy_j - x_j r^3 (1/D) sum_k x_k w_k dy_k,   dw_j = sum over tokens of x_j r dy_j.
    """
    d = x.shape[-1]
    h = d // 2
    g1, g2 = g[..., :h], g[..., h:]
    dy = np.concatenate([g1 * cos + g2 * sin, -g1 * sin + g2 * cos], axis=-1)
    if w is None:
        return dy, None
    wdy = w * dy
    dx = r[..., None] * wdy - x * (r ** 3)[..., None] * (np.sum(x * wdy, axis=-1) / d)[..., None]
    dw = None if w is None else np.sum((x * r[..., None] * dy).reshape(-1, d), axis=0)
    return dx, dw


def prefill_forward_backward(q_bits, k_bits, v_bits, q_norm_weight, k_norm_weight, positions, dout_bits,
                             *, eps: float = 1e-6, theta: float = 1e6, scale: float = 1.0, exact_inputs=None):
    """Forward (out, lse) and gradients (dq, dk, dv, dq_norm_weight, dk_norm_weight) in float64.

    q_bits [B, Hq, S, D], k_bits, v_bits [B, Hkv, S, D], dout_bits [B, Hq, S, D]: BF16 bit
    patterns (uint16).  positions [B, S].  Norm weights float32 [D] or None.
    ``exact_inputs``: optional dict of float64 arrays {q, k, v, dout, wq, wk} used instead of the
    BF16 inputs, with q^ and k^ in exact arithmetic (no rounding anywhere), so the function is
    smooth (for finite-difference checks of the gradients).
    Query head h reads KV head h // (Hq / Hkv).  Softmax scale 1/sqrt(D).
    """
    if exact_inputs is None:
        q = f32_from_bf16_bits(q_bits).astype(np.float64)
        k = f32_from_bf16_bits(k_bits).astype(np.float64)
        v = f32_from_bf16_bits(v_bits).astype(np.float64)
        do = f32_from_bf16_bits(dout_bits).astype(np.float64)
        wq = None if q_norm_weight is None else np.asarray(q_norm_weight, dtype=np.float64)
        wk = None if k_norm_weight is None else np.asarray(k_norm_weight, dtype=np.float64)
    else:
        q, k, v, do = (np.asarray(exact_inputs[n], dtype=np.float64) for n in ("q", "k", "v", "dout"))
        wq, wk = exact_inputs.get("wq"), exact_inputs.get("wk")
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    c = 1.0 / math.sqrt(D)
    pos = np.asarray(positions, dtype=np.int64)
    out = np.zeros_like(q)
    lse = np.zeros((B, Hq, S))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dwq = None if wq is None else np.zeros(D)
    dwk = None if wk is None else np.zeros(D)
    for b in range(B):
        cs, sn = (a.astype(np.float64) for a in rope_cos_sin(pos[b], D, theta, scale))  # [S, D/2]
        visible = pos[b][None, :] <= pos[b][:, None]                                   # [query, key]
        def boundary(bits, x, w):
            """q^ or k^: exact, or the forward reference's post-RoPE BF16 values"""
            exact, r = _norm_rope_forward(x, w, cs, sn, eps)
            if exact_inputs is not None:
                return exact, r
            wf = None if w is None else np.asarray(w, dtype=np.float32)
            return prologue(bits, wf, pos[b], eps, theta, scale).astype(np.float64), r

        for hk in range(Hkv):
            khat, rk = boundary(None if k_bits is None else k_bits[b, hk], k[b, hk], wk)
            dkhat = np.zeros((S, D))
            for h in range(hk * G, (hk + 1) * G):
                qhat, rq = boundary(None if q_bits is None else q_bits[b, h], q[b, h], wq)
                s = np.where(visible, (qhat @ khat.T) * c, -np.inf)
                m = np.max(s, axis=1, keepdims=True)
                p = np.exp(s - m)
                tot = np.sum(p, axis=1, keepdims=True)
                p = p / tot
                o = p @ v[b, hk]
                out[b, h] = o
                lse[b, h] = (m + np.log(tot))[:, 0]
                dp = do[b, h] @ v[b, hk].T
                dsc = p * (dp - np.sum(do[b, h] * o, axis=1, keepdims=True))
                dv[b, hk] += p.T @ do[b, h]
                dqhat = c * (dsc @ khat)
                dkhat += c * (dsc.T @ qhat)
                gq, gwq = _norm_rope_backward(q[b, h], wq, cs, sn, rq, dqhat)
                dq[b, h] = gq
                if dwq is not None:
                    dwq += gwq
            gk, gwk = _norm_rope_backward(k[b, hk], wk, cs, sn, rk, dkhat)
            dk[b, hk] = gk
            if dwk is not None:
                dwk += gwk
    return out, lse, dq, dk, dv, dwq, dwk
