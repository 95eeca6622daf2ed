"""Pins of the backward reference (oracle/backward.py): central finite differences of the
exact-arithmetic forward it differentiates, on small inputs, for every input it returns a
gradient for; and its forward against the forward reference of oracle/definition.py."""

import math

import numpy as np
import pytest

import oracle
from oracle.backward import prefill_forward_backward

D = 16


def _exact_inputs(rng, B=1, Hq=4, Hkv=2, S=5):
    return dict(q=rng.standard_normal((B, Hq, S, D)), k=rng.standard_normal((B, Hkv, S, D)),
                v=rng.standard_normal((B, Hkv, S, D)), dout=rng.standard_normal((B, Hq, S, D)),
                wq=rng.uniform(0.5, 1.5, D), wk=rng.uniform(0.5, 1.5, D))


def test_gradients_without_norm_match_central_differences():
    """No norm weights: the prologue is the rotation alone (as the forward reference skips the
    RMSNorm when the weight is None)."""
    rng = np.random.default_rng(12)
    inp = _exact_inputs(rng)
    inp["wq"] = inp["wk"] = None
    pos = np.array([[0, 1, 2, 3, 4]])
    _, _, dq, dk, dv, dwq, dwk = prefill_forward_backward(None, None, None, None, None, pos, None, exact_inputs=inp)
    assert dwq is None and dwk is None
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        flat = inp[name].reshape(-1)
        for i in rng.choice(flat.size, size=20, replace=False):
            keep = flat[i]
            flat[i] = keep + 1e-6
            up = _loss(inp, pos)
            flat[i] = keep - 1e-6
            dn = _loss(inp, pos)
            flat[i] = keep
            fd = (up - dn) / 2e-6
            assert abs(fd - grad.reshape(-1)[i]) <= 1e-6 * max(1.0, abs(fd)), (name, int(i))


def _loss(inp, pos):
    out = prefill_forward_backward(None, None, None, None, None, pos, None, exact_inputs=inp)[0]
    return float(np.sum(out * inp["dout"]))


@pytest.mark.parametrize("name", ["q", "k", "v", "wq", "wk"])
def test_gradients_match_central_differences(name):
    rng = np.random.default_rng(11)
    inp = _exact_inputs(rng)
    pos = np.array([[0, 1, 2, 4, 7]])  # not contiguous: visibility follows the positions
    _, _, dq, dk, dv, dwq, dwk = prefill_forward_backward(None, None, None, None, None, pos, None, exact_inputs=inp)
    grad = {"q": dq, "k": dk, "v": dv, "wq": dwq, "wk": dwk}[name]
    x = inp[name]
    flat = x.reshape(-1)
    h = 1e-6
    idx = rng.choice(flat.size, size=min(40, flat.size), replace=False)
    for i in idx:
        keep = flat[i]
        flat[i] = keep + h
        up = _loss(inp, pos)
        flat[i] = keep - h
        dn = _loss(inp, pos)
        flat[i] = keep
        fd = (up - dn) / (2 * h)
        g = grad.reshape(-1)[i]
        assert abs(fd - g) <= 1e-6 * max(1.0, abs(fd)), (name, int(i), fd, g)


def test_forward_matches_the_forward_reference():
    """On BF16 inputs the backward's forward is the forward reference (the same post-RoPE BF16
    q^ and k^, float64 attention), up to the reference's final roundings of out and lse."""
    rng = np.random.default_rng(3)
    B, Hq, Hkv, S, Dm = 1, 2, 1, 6, 128
    bits = lambda shape: oracle.bf16_bits_from_f32(rng.standard_normal(shape).astype(np.float32))
    q, k, v, do = bits((B, Hq, S, Dm)), bits((B, Hkv, S, Dm)), bits((B, Hkv, S, Dm)), bits((B, Hq, S, Dm))
    wq = rng.uniform(0.5, 1.5, Dm).astype(np.float32)
    wk = rng.uniform(0.5, 1.5, Dm).astype(np.float32)
    pos = np.arange(S)[None]
    out, lse = prefill_forward_backward(q, k, v, wq, wk, pos, do)[:2]
    # the same problem through the paged forward reference: one page-size-16 page holding the row
    kc = np.zeros((1, 16, Hkv, Dm), dtype=np.uint16)
    vc = np.zeros((1, 16, Hkv, Dm), dtype=np.uint16)
    kc[0, :S] = np.transpose(k[0], (1, 0, 2))
    vc[0, :S] = np.transpose(v[0], (1, 0, 2))
    ref_bits, ref_lse = oracle.paged_attention(q, kc, vc, np.array([0, 1]), np.array([0]), np.array([S]), pos,
                                               np.arange(16), wq, wk)
    ref = oracle.f32_from_bf16_bits(ref_bits).astype(np.float64)
    # the same q^, k^ and float64 attention: out differs only by the reference's BF16 rounding
    # (half an ulp of an 8-bit significand: 2^-8 relative), lse by its float32 rounding
    assert np.all(np.abs(ref - out) <= 2.0 ** -8 * np.abs(out) + 1e-30)
    assert np.all(np.abs(ref_lse - lse) <= 2.0 ** -23 * np.abs(lse) + 1e-30)


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 1)])
def test_gradients_other_groups_and_two_rows(Hq, Hkv):
    """GQA groups 1 and 4 with two rows at different positions: the head-to-KV-head map and the
    per-row sums, against central differences of q, k and v."""
    rng = np.random.default_rng(20 + Hq)
    inp = _exact_inputs(rng, B=2, Hq=Hq, Hkv=Hkv, S=4)
    pos = np.array([[0, 1, 2, 3], [3, 0, 5, 1]])
    _, _, dq, dk, dv, _, _ = prefill_forward_backward(None, None, None, None, None, pos, None, exact_inputs=inp)
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        flat = inp[name].reshape(-1)
        for i in rng.choice(flat.size, size=15, replace=False):
            keep = flat[i]
            flat[i] = keep + 1e-6
            up = _loss(inp, pos)
            flat[i] = keep - 1e-6
            dn = _loss(inp, pos)
            flat[i] = keep
            fd = (up - dn) / 2e-6
            assert abs(fd - grad.reshape(-1)[i]) <= 1e-6 * max(1.0, abs(fd)), (name, int(i))
