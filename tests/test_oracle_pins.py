"""Pins for the CPU oracle: closed forms, library routines, brute force and invariants.

None of these tests re-types the oracle's formulas; each checks it against
something fixed independently of it (mathematics, torch/numpy library
routines, exact rational arithmetic, or a brute-force construction), chosen so
that a dropped term, a wrong sign or index, or a transposed operand anywhere in
the oracle fails at least one of them.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import definition as pa
import workloads

D = 128


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _bf16_from_torch(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------------------------------------
# BF16 encoding
# ---------------------------------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    rng = _rng(1)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),  # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], np.float32),
    ])
    # ties: random bf16 values plus exactly half a bf16 ulp
    base = _bf16_from_torch(rng.standard_normal(10000).astype(np.float32)).astype(np.uint32) << 16
    ties = (base | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties])
    np.testing.assert_array_equal(oracle.bf16_bits_from_f32(x), _bf16_from_torch(x))
    assert oracle.bf16_bits_from_f32(np.array([np.nan], np.float32))[0] == 0x7FC0


def test_bf16_widening_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    got = oracle.f32_from_bf16_bits(bits)
    np.testing.assert_array_equal(got[finite], ref[finite])


def _exact_bf16_round(x: float) -> float:
    """Correct RNE rounding of a finite float64 to BF16 by exact rational comparison."""
    if x == 0:
        return x
    f = Fraction(x)
    sign = -1 if f < 0 else 1
    a = abs(f)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 7)
    lo = (a // ulp) * ulp
    hi = lo + ulp
    if a - lo < hi - a:
        r = lo
    elif a - lo > hi - a:
        r = hi
    else:
        r = lo if (lo / ulp) % 2 == 0 else hi
    return float(sign * r)


def test_bf16_from_f64_single_rounding():
    rng = _rng(2)
    vals = []
    # values just off a BF16 midpoint by less than a float32 ulp: a float64 -> float32 -> bf16
    # chain rounds these the wrong way
    for _ in range(400):
        m = _bf16_from_torch(np.array([rng.standard_normal()], np.float32)).astype(np.uint32)[0] << 16
        mid = float((m | np.uint32(0x8000)).view(np.float32))
        ulp32 = abs(float(np.spacing(np.float32(mid))))
        vals.append(mid + rng.uniform(-0.49, 0.49) * ulp32)
        vals.append(mid)
    vals += list(rng.standard_normal(2000))
    got = oracle.f32_from_bf16_bits(oracle.bf16_bits_from_f64(np.array(vals)))
    ref = np.array([_exact_bf16_round(v) for v in vals], np.float32)
    np.testing.assert_array_equal(got, ref)


# ---------------------------------------------------------------------------------------------
# Paged geometry
# ---------------------------------------------------------------------------------------------

def test_row_lengths_closed_form():
    indptr = np.array([0, 3, 3, 5, 6])
    last = np.array([7, 1, 16, 1])
    np.testing.assert_array_equal(oracle.row_lengths(indptr, last, 16), [2 * 16 + 7, 0, 16 + 16, 1])


def test_logical_kv_inverts_a_scatter():
    """Scatter a dense logical K/V into random pages, then gather it back."""
    rng = _rng(3)
    lengths = [37, 0, 16, 1, 80]
    num_pages = 40
    order = rng.permutation(num_pages).astype(np.int32)
    indptr, indices, last, _ = workloads.csr_from_lengths(lengths, order)
    hkv = 3
    kc = np.zeros((num_pages, 16, hkv, 4), np.uint16)
    vc = np.zeros_like(kc)
    dense = {}
    for b, L in enumerate(lengths):
        dk = rng.integers(1, 60000, (L, hkv, 4)).astype(np.uint16)
        dv = rng.integers(1, 60000, (L, hkv, 4)).astype(np.uint16)
        dense[b] = (dk, dv)
        for j in range(L):  # brute-force scatter, one key at a time
            page = indices[indptr[b] + j // 16]
            kc[page, j % 16] = dk[j]
            vc[page, j % 16] = dv[j]
    for b in range(len(lengths)):
        k, v = oracle.logical_kv(kc, vc, indptr, indices, last, b, 16)
        np.testing.assert_array_equal(k, dense[b][0])
        np.testing.assert_array_equal(v, dense[b][1])


# ---------------------------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------------------------

def _bf16_vectors(seed, n):
    return oracle.f32_from_bf16_bits(workloads.bf16_normal(_rng(seed), (n, D)))


def test_rmsnorm_sum_of_squares_is_exact():
    """ms must equal RN32(exact sum / D): checked with math.fsum (exact float summation)."""
    x = _bf16_vectors(4, 300)
    w = np.ones(D, np.float32)
    y = oracle.rmsnorm_fp32(x, w, 0.0)
    for r in range(x.shape[0]):
        ss = math.fsum(float(v) * float(v) for v in x[r])
        ms = np.float32(ss / D)
        inv = np.float32(1.0 / math.sqrt(float(ms)))
        np.testing.assert_array_equal(y[r], x[r] * inv)


def test_rmsnorm_unit_rms_and_torch():
    rng = _rng(5)
    x = _bf16_vectors(5, 500)
    w = rng.uniform(0.5, 1.5, D).astype(np.float32)
    y = oracle.rmsnorm_fp32(x, w, 1e-6).astype(np.float64)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x.astype(np.float64)), (D,),
                                       torch.from_numpy(w.astype(np.float64)), 1e-6).numpy()
    np.testing.assert_allclose(y, ref, rtol=3e-7, atol=1e-30)
    y1 = oracle.rmsnorm_fp32(x, np.ones(D, np.float32), 0.0).astype(np.float64)
    np.testing.assert_allclose(np.sqrt(np.mean(y1 ** 2, axis=-1)), 1.0, rtol=1e-6)


def test_rmsnorm_scale_invariance():
    x = _bf16_vectors(6, 200)
    w = _rng(6).uniform(0.5, 1.5, D).astype(np.float32)
    a = oracle.rmsnorm_fp32(x, w, 0.0)
    b = oracle.rmsnorm_fp32(x * np.float32(8.0), w, 0.0)  # power-of-two scaling is exact
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------------------------

def test_rope_inv_freq_closed_forms():
    f = pa.rope_inv_freq(D, 1e6)
    assert f[0] == 1.0
    assert abs(f[32] - 1e-3) <= 2e-19              # (1e6)^(-1/2)
    assert abs(f[16] - 10 ** -1.5) <= 1e-17        # (1e6)^(-1/4)
    assert np.all(np.diff(f) < 0)


def test_rope_cos_sin_closed_forms():
    c, s = oracle.rope_cos_sin(np.array([0, 1, 131071]), D, 1e6, 1.0)
    assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)
    assert c[1, 0] == np.float32(math.cos(1.0)) and s[1, 0] == np.float32(math.sin(1.0))
    assert c[2, 0] == np.float32(math.cos(131071.0)) and s[2, 0] == np.float32(math.sin(131071.0))
    # frequency 32 is 1e-3 rad per position
    assert abs(float(c[2, 32]) - math.cos(131.071)) < 1e-7
    # rope_scale divides the position
    c2, s2 = oracle.rope_cos_sin(np.array([2]), D, 1e6, 2.0)
    assert c2[0, 0] == np.float32(math.cos(1.0))


def test_rope_pairing_and_sign():
    """A unit vector along dim i rotates into dim i + D/2 with +sin (rotate-half convention)."""
    ang = 0.7
    c = np.full((1, D // 2), np.cos(ang), np.float32)
    s = np.full((1, D // 2), np.sin(ang), np.float32)
    for i in (0, 5, 63):
        e = np.zeros((1, D), np.float32)
        e[0, i] = 1.0
        r = oracle.rope_fp32(e, c, s)
        assert r[0, i] == c[0, 0] and r[0, i + 64] == s[0, 0]
        assert np.count_nonzero(r) == 2
        e = np.zeros((1, D), np.float32)
        e[0, i + 64] = 1.0
        r = oracle.rope_fp32(e, c, s)
        assert r[0, i] == -s[0, 0] and r[0, i + 64] == c[0, 0]


def test_rope_matches_complex_rotation():
    rng = _rng(7)
    y = rng.standard_normal((50, D)).astype(np.float32)
    pos = rng.integers(0, 140000, 50)
    c, s = oracle.rope_cos_sin(pos, D, 1e6, 1.0)
    got = oracle.rope_fp32(y, c, s).astype(np.float64)
    z = (y[:, :64].astype(np.float64) + 1j * y[:, 64:].astype(np.float64)) * \
        np.exp(1j * pos[:, None] * pa.rope_inv_freq(D, 1e6)[None, :])
    np.testing.assert_allclose(got[:, :64], z.real, atol=2e-6)
    np.testing.assert_allclose(got[:, 64:], z.imag, atol=2e-6)


def test_rope_relative_position_property():
    rng = _rng(8)
    q = rng.standard_normal((20, D)).astype(np.float32)
    k = rng.standard_normal((20, D)).astype(np.float32)
    p, pk, delta = 700, 200, 5000
    def rot(x, pos):
        c, s = oracle.rope_cos_sin(np.full(x.shape[0], pos), D, 1e6, 1.0)
        return oracle.rope_fp32(x, c, s).astype(np.float64)
    a = np.sum(rot(q, p) * rot(k, pk), axis=-1)
    b = np.sum(rot(q, p + delta) * rot(k, pk + delta), axis=-1)
    np.testing.assert_allclose(a, b, atol=2e-4)
    # pair norms are preserved
    r = rot(q, 12345)
    np.testing.assert_allclose(r[:, :64] ** 2 + r[:, 64:] ** 2,
                               q[:, :64].astype(np.float64) ** 2 + q[:, 64:].astype(np.float64) ** 2,
                               rtol=1e-6)


def test_prologue_at_position_zero_is_rmsnorm_only():
    bits = workloads.bf16_normal(_rng(9), (30, D))
    w = _rng(9).uniform(0.5, 1.5, D).astype(np.float32)
    got = oracle.prologue(bits, w, np.zeros(30, np.int64), 1e-6, 1e6, 1.0)
    want = oracle.bf16_round(oracle.rmsnorm_fp32(oracle.f32_from_bf16_bits(bits), w, 1e-6))
    np.testing.assert_array_equal(got, want)
    # no weight -> no norm: pure RoPE of the raw values
    got = oracle.prologue(bits, None, np.zeros(30, np.int64), 1e-6, 1e6, 1.0)
    np.testing.assert_array_equal(got, oracle.f32_from_bf16_bits(bits))


# ---------------------------------------------------------------------------------------------
# Attention core
# ---------------------------------------------------------------------------------------------

def test_attention_zero_query_closed_form():
    """q = 0: all scores 0, so LSE = ln(#visible) and out = mean of the visible values."""
    rng = _rng(10)
    L, Sq = 45, 6
    v = rng.standard_normal((L, D))
    qpos = np.arange(L - Sq, L)
    out, lse = oracle.attention_fp64(np.zeros((2, Sq, D)), rng.standard_normal((L, D)), v,
                                     qpos, np.arange(L), 1 / math.sqrt(D))
    for i, p in enumerate(qpos):
        n = p + 1
        np.testing.assert_allclose(lse[:, i], math.log(n), rtol=0, atol=1e-14)
        np.testing.assert_allclose(out[:, i], np.broadcast_to(v[:n].mean(0), (2, D)), atol=1e-13)


def test_attention_single_key():
    rng = _rng(11)
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, D))
    v = rng.standard_normal((1, D))
    out, lse = oracle.attention_fp64(q, k, v, np.array([5]), np.array([0]), 0.125)
    np.testing.assert_array_equal(out[0, 0], v[0])
    assert abs(lse[0, 0] - float(q[0, 0] @ k[0]) * 0.125) < 1e-13


def test_attention_no_visible_keys():
    out, lse = oracle.attention_fp64(np.ones((1, 2, D)), np.ones((3, D)), np.ones((3, D)),
                                     np.array([-1, -1]), np.arange(3), 0.1)
    assert np.all(out == 0) and np.all(lse == -np.inf)
    out, lse = oracle.attention_fp64(np.ones((1, 1, D)), np.zeros((0, D)), np.zeros((0, D)),
                                     np.array([0]), np.arange(0), 0.1)
    assert np.all(out == 0) and np.all(lse == -np.inf)


def test_attention_matches_torch_sdpa_and_logsumexp():
    rng = _rng(12)
    L, Sq, G = 70, 9, 3
    q = rng.standard_normal((G, Sq, D))
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    qpos = np.arange(L - Sq, L)
    out, lse = oracle.attention_fp64(q, k, v, qpos, np.arange(L), 1 / math.sqrt(D))
    mask = torch.from_numpy(np.arange(L)[None, :] <= qpos[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k)[None].expand(G, L, D),
        torch.from_numpy(v)[None].expand(G, L, D), attn_mask=mask)
    np.testing.assert_allclose(out, ref.numpy(), atol=1e-12)
    scores = torch.from_numpy(q) @ torch.from_numpy(k).T / math.sqrt(D)
    scores = scores.masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(scores, dim=-1).numpy(), atol=1e-12)


def test_attention_brute_force_tiny():
    """Pure-Python loops with math.exp on a 2-query, 5-key, 4-dim problem."""
    rng = _rng(13)
    d, L = 4, 5
    q = rng.standard_normal((1, 2, d))
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    qpos = [2, 4]
    out, lse = oracle.attention_fp64(q, k, v, np.array(qpos), np.arange(L), 0.5)
    for i, p in enumerate(qpos):
        s = [sum(q[0, i, t] * k[j, t] for t in range(d)) * 0.5 for j in range(p + 1)]
        z = sum(math.exp(x) for x in s)
        assert abs(lse[0, i] - math.log(z)) < 1e-13
        for t in range(d):
            o = sum(math.exp(s[j]) / z * v[j, t] for j in range(p + 1))
            assert abs(out[0, i, t] - o) < 1e-13


# ---------------------------------------------------------------------------------------------
# Whole paged path
# ---------------------------------------------------------------------------------------------

def _small_batch(seed=20, lengths=(37, 16, 1, 90), q_len=1, hq=8, hkv=2, mode="decode", pages=64):
    return workloads.make_batch(seed, list(lengths), q_len=q_len, num_q_heads=hq, num_kv_heads=hkv,
                                num_pages=pages, query_mode=mode)


def _run(b, **kw):
    args, kwargs = b.oracle_args()
    kwargs.update(kw)
    return oracle.paged_attention(*args, **kwargs)


def test_paged_zero_query_gives_prefix_means():
    """q = 0 pins paging, logical order and the causal mask in one check."""
    b = _small_batch(lengths=(40, 33), q_len=5, mode="prefill")
    b.q[:] = 0
    out, lse = _run(b)
    for r in range(b.batch):
        kb, vb = oracle.logical_kv(b.k_cache, b.v_cache, b.kv_indptr, b.kv_indices, b.kv_last_page_len, r, 16)
        v = oracle.f32_from_bf16_bits(vb).astype(np.float64)
        for i, p in enumerate(b.query_position_ids[r]):
            n = int(p) + 1
            np.testing.assert_allclose(lse[r, :, i], math.log(n), atol=1e-6)
            for h in range(b.num_q_heads):
                # out must be a BF16 rounding (within half an ulp, up to 1e-12 of float64
                # evaluation-order slack) of the exact mean of the visible values
                mean = v[:n, h // 4].mean(0)
                got = oracle.f32_from_bf16_bits(out[r, h, i]).astype(np.float64)
                ulp = 2.0 ** (np.floor(np.log2(np.abs(mean))) - 7)
                assert np.all(np.abs(got - mean) <= 0.5 * ulp + 1e-12 * np.abs(mean))


def test_paged_matches_dense_sdpa_on_materialised_inputs():
    """The paged path equals float64 SDPA on the logical q^, k^, v built by brute force."""
    b = _small_batch(lengths=(50, 17), q_len=4, mode="prefill")
    out, lse = _run(b)
    G = b.num_q_heads // b.num_kv_heads
    for r in range(b.batch):
        L = int(b.lengths[r])
        qpos = b.query_position_ids[r]
        kpos = np.arange(L)
        for h in range(b.num_q_heads):
            hk = h // G
            keys = []
            vals = []
            for j in range(L):
                page = b.kv_indices[b.kv_indptr[r] + j // 16]
                keys.append(b.k_cache[page, j % 16, hk])
                vals.append(b.v_cache[page, j % 16, hk])
            kh = oracle.prologue(np.stack(keys), b.k_norm_weight, kpos, 1e-6, 1e6, 1.0).astype(np.float64)
            qh = oracle.prologue(b.q[r, h], b.q_norm_weight, qpos, 1e-6, 1e6, 1.0).astype(np.float64)
            vv = oracle.f32_from_bf16_bits(np.stack(vals)).astype(np.float64)
            mask = torch.from_numpy(kpos[None, :] <= qpos[:, None])
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qh)[None], torch.from_numpy(kh)[None], torch.from_numpy(vv)[None],
                attn_mask=mask)[0].numpy()
            np.testing.assert_array_equal(out[r, h], oracle.bf16_bits_from_f64(ref))
            sc = torch.from_numpy(qh) @ torch.from_numpy(kh).T / math.sqrt(D)
            ref_lse = torch.logsumexp(sc.masked_fill(~mask, float("-inf")), -1).numpy().astype(np.float32)
            np.testing.assert_allclose(lse[r, h], ref_lse, rtol=0, atol=2e-7)


def test_paged_gqa_equals_repeated_mha():
    b = _small_batch(lengths=(29, 64), hq=8, hkv=2)
    out_gqa, lse_gqa = _run(b)
    G = 4
    mha = workloads.PagedBatch(**{**b.__dict__,
                                  "k_cache": np.repeat(b.k_cache, G, axis=2),
                                  "v_cache": np.repeat(b.v_cache, G, axis=2)})
    out_mha, lse_mha = _run(mha)
    np.testing.assert_array_equal(out_gqa, out_mha)
    np.testing.assert_array_equal(lse_gqa, lse_mha)


def test_paged_page_permutation_invariance():
    b = _small_batch(lengths=(37, 16, 1, 90))
    p = workloads.permute_pages(b, 99)
    assert not np.array_equal(p.kv_indices, b.kv_indices)
    o1, l1 = _run(b)
    o2, l2 = _run(p)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_paged_row_alone_equals_row_in_batch():
    full = workloads.invariance_batch(alone=False, num_pages=8192)
    alone = workloads.invariance_batch(alone=True, num_pages=8192)
    r = workloads.INVARIANCE_ROW_INDEX
    o1, l1 = _run(full, rows=[r], q_heads=[0, 9, 31])
    o2, l2 = _run(alone, rows=[0], q_heads=[0, 9, 31])
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_paged_empty_row_and_subset_selection():
    b = _small_batch(lengths=(20, 0, 33))
    out, lse = _run(b)
    assert np.all(out[1] == 0) and np.all(lse[1] == -np.inf)
    assert np.all(np.isfinite(lse[[0, 2]]))
    o, l = _run(b, rows=[2, 0], q_heads=[7, 1])
    np.testing.assert_array_equal(o[0, 0], out[2, 7])
    np.testing.assert_array_equal(l[1, 1], lse[0, 1])


def test_paged_canaries_never_reach_the_result():
    b = _small_batch(lengths=(37, 16, 1, 90))
    assert np.any(b.k_cache == 0x7FC0)
    out, lse = _run(b)
    assert np.all(np.isfinite(lse))
    assert not np.any(np.isnan(oracle.f32_from_bf16_bits(out)))


# ---------------------------------------------------------------------------------------------
# The prologue's composition at non-zero positions.  "WS2 Attention Cross-Configuration
# Integration", section "H100 Attention input and projection boundary": inside the attention
# boundary the order is Q/K RMSNorm, then RoPE; "[WS2][PR7][Attention] Add FlashInfer
# RoPE-fused paged attention scaffold", section "Scope": both sides share the post-RoPE BF16
# boundary.  RMSNorm's scale factor is rotation-invariant, so what these pins catch is where
# the per-dimension weight sits: applied before the rotation (correct), after it, or the two
# operations swapped, all differ as soon as w_i != w_{i+64}.
# ---------------------------------------------------------------------------------------------

def _independent_prologue64(x_bits, w, pos):
    """RMSNorm by torch's float64 rms_norm (with the weight), then the rotation as a complex
    product (y_i + i y_{i+64}) * exp(i pos theta^(-2i/128)); float64, no rounding."""
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).to(torch.float64)
    if w is not None:
        x = torch.nn.functional.rms_norm(x, (D,), torch.from_numpy(np.asarray(w, np.float64)), 1e-6)
    freq = torch.tensor([1e6 ** (-2.0 * i / D) for i in range(D // 2)], dtype=torch.float64)
    ang = torch.from_numpy(np.asarray(pos, np.float64))[:, None] * freq[None, :]
    z = torch.complex(x[:, :D // 2], x[:, D // 2:]) * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([z.real, z.imag], dim=-1).numpy()


def _bf16_half_ulp(v):
    """Half a BF16 ulp at |v| (the rounding error the post-RoPE cast may add)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 0.5 * np.exp2(np.floor(np.log2(a)) - 7)


@pytest.mark.parametrize("with_weight", [True, False])
def test_prologue_matches_independent_norm_then_rotation(with_weight):
    """oracle.prologue at random positions up to 131,071 equals the independent float64
    construction rounded to BF16: within half a BF16 ulp plus FP32 evaluation slack."""
    rng = _rng(31)
    n = 600
    bits = workloads.bf16_normal(rng, (n, D))
    w = rng.uniform(0.5, 1.5, D).astype(np.float32) if with_weight else None
    pos = np.concatenate([rng.integers(1, 131072, n - 4), [1, 4095, 65536, 131071]])
    got = oracle.prologue(bits, w, pos, 1e-6, 1e6, 1.0).astype(np.float64)
    ref = _independent_prologue64(bits, w, pos)
    # FP32 slack: the prologue's few float32 roundings and the float32 cos/sin, relative to
    # the pair's magnitude
    pair = np.sqrt(ref[:, :64] ** 2 + ref[:, 64:] ** 2)
    slack = 2.0 ** -20 * np.concatenate([pair, pair], axis=-1)
    assert np.all(np.abs(got - ref) <= _bf16_half_ulp(ref) + slack)
    # the planted mistakes: the weight after the rotation, and the two operations swapped
    if with_weight:
        x = oracle.f32_from_bf16_bits(bits)
        c, s = oracle.rope_cos_sin(pos, D, 1e6, 1.0)
        w_after = oracle.bf16_round(oracle.rope_fp32(oracle.rmsnorm_fp32(x, np.ones(D, np.float32), 1e-6), c, s) * w)
        swapped = oracle.bf16_round(oracle.rmsnorm_fp32(oracle.rope_fp32(x, c, s), w, 1e-6))
        for wrong in (w_after, swapped):
            assert np.max(np.abs(wrong.astype(np.float64) - ref)) > 0.05


def test_prologue_one_hot_closed_form():
    """x = a e_i (one-hot at dim i < 64) at position p: RMSNorm gives y_i = w_i a r with
    r = 1/sqrt(a^2/128 + eps) and zero elsewhere, and the rotation sends it to dims i and i+64
    as (y_i cos, y_i sin) of frequency i.  The weight of dim i+64 must not appear."""
    rng = _rng(32)
    w = rng.uniform(0.5, 1.5, D).astype(np.float32)
    for i, p, a in ((0, 1, 1.5), (7, 1000, -2.0), (40, 77777, 0.75), (63, 131071, 3.0)):
        x = np.zeros((1, D), np.float32)
        x[0, i] = a
        bits = oracle.bf16_bits_from_f32(x)
        got = oracle.prologue(bits, w, np.array([p]), 1e-6, 1e6, 1.0)[0].astype(np.float64)
        r = 1.0 / math.sqrt(a * a / D + 1e-6)
        ang = p * 1e6 ** (-2.0 * i / D)
        want_i = float(w[i]) * a * r * math.cos(ang)
        want_j = float(w[i]) * a * r * math.sin(ang)
        for got_v, want in ((got[i], want_i), (got[i + 64], want_j)):
            assert abs(got_v - want) <= _bf16_half_ulp(np.array(want)) + 2.0 ** -20 * abs(a * r * 1.5)
        assert np.count_nonzero(got) == 2 - (got[i + 64] == 0) - (got[i] == 0)


def test_backward_exact_prologue_matches_independent_construction():
    """oracle/backward.py's exact-arithmetic prologue (the function its gradients
    differentiate) against the same independent float64 construction, at non-zero positions.
    Its cos/sin are the float32 ones, so agreement is to ~2^-23 of the pair magnitude."""
    from oracle.backward import _norm_rope_forward

    rng = _rng(33)
    n = 200
    bits = workloads.bf16_normal(rng, (n, D))
    w = rng.uniform(0.5, 1.5, D).astype(np.float32)
    pos = rng.integers(1, 131072, n)
    x = oracle.f32_from_bf16_bits(bits).astype(np.float64)
    c, s = (a.astype(np.float64) for a in oracle.rope_cos_sin(pos, D, 1e6, 1.0))
    for wt in (w, None):
        got, _ = _norm_rope_forward(x, None if wt is None else wt.astype(np.float64), c, s, 1e-6)
        ref = _independent_prologue64(bits, wt, pos)
        pair = np.sqrt(ref[:, :64] ** 2 + ref[:, 64:] ** 2)
        np.testing.assert_array_less(np.abs(got - ref), 2.0 ** -21 * np.concatenate([pair, pair], -1) + 1e-300)
