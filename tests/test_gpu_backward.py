"""pa_prefill_backward on the GPU against the CPU oracle's gradients, bitwise repeatability,
and row-local results (a row alone has the same dq, dk, dv bits as inside a batch).

Tolerance.  The kernels feed the matrix cores BF16 operands: q^, k^, v, dout (exact inputs)
and P and dS rounded to BF16 (relative error <= 2^-8 each), and use the forward's BF16 out
in Dv = sum dout * out.  Each gradient entry is a sum of such terms with FP32 accumulation, so
its error is a few 2^-8 of the terms' magnitude; the gates below are 2e-2 of each tensor's
largest entry (max-abs, plus 1e-4 absolute) and 1e-2 of its Frobenius norm.
"""

import numpy as np
import pytest
import torch

import oracle
import deterministic_paged_kv_amd as pa
from _paged import bf16_tensor, i32

pytestmark = pytest.mark.gpu


def _case(seed, B, Hq, Hkv, S, norm=True):
    rng = np.random.default_rng(seed)
    bits = lambda shape: oracle.bf16_bits_from_f32(rng.standard_normal(shape).astype(np.float32))
    q, k, v, do = bits((B, Hq, S, 128)), bits((B, Hkv, S, 128)), bits((B, Hkv, S, 128)), bits((B, Hq, S, 128))
    wq = rng.uniform(0.5, 1.5, 128).astype(np.float32) if norm else None
    wk = rng.uniform(0.5, 1.5, 128).astype(np.float32) if norm else None
    pos = np.tile(np.arange(S, dtype=np.int32), (B, 1))
    return q, k, v, do, wq, wk, pos


def _forward(plan, q, k, v, wq, wk, pos):
    """pa_prefill on the dense inputs laid out in pages (row b's tokens in its own pages)."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    npg = (S + 15) // 16
    kc = np.zeros((B * npg, 16, Hkv, D), dtype=np.uint16)
    vc = np.zeros((B * npg, 16, Hkv, D), dtype=np.uint16)
    for b in range(B):
        for t in range(S):
            kc[b * npg + t // 16, t % 16] = k[b, :, t]
            vc[b * npg + t // 16, t % 16] = v[b, :, t]
    indptr = np.arange(B + 1, dtype=np.int32) * npg
    indices = np.arange(B * npg, dtype=np.int32)
    last = np.full(B, S - (npg - 1) * 16, dtype=np.int32)
    f = lambda a: None if a is None else torch.from_numpy(a).cuda()
    kpos = np.tile(np.arange(npg * 16, dtype=np.int32), B)  # key j of row b at b * npg * 16 + j
    out, lse = pa.prefill(plan, bf16_tensor(q), bf16_tensor(kc), bf16_tensor(vc), i32(indptr), i32(indices), i32(last),
                          i32(pos), i32(pos), i32(kpos), f(wq), f(wk))
    return out, lse


def _run(seed, B, Hq, Hkv, S, norm=True, repeats=1):
    q, k, v, do, wq, wk, pos = _case(seed, B, Hq, Hkv, S, norm)
    plan = pa.Plan(Hq, Hkv, max_batch=B, max_q_len=S, max_pages_per_row=(S + 15) // 16)
    out, lse = _forward(plan, q, k, v, wq, wk, pos)
    f = lambda a: None if a is None else torch.from_numpy(a).cuda()
    args = (i32(pos), bf16_tensor(q), bf16_tensor(k), bf16_tensor(v), out, lse, bf16_tensor(do))
    results = []
    for _ in range(repeats):
        g = pa.prefill_backward(plan, *args, q_norm_weight=f(wq), k_norm_weight=f(wk))
        torch.cuda.synchronize()
        results.append([None if t is None else t.cpu().numpy() for t in g])
    return (q, k, v, do, wq, wk, pos), results


def _check(name, got, ref):
    scale = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(got.astype(np.float64) - ref)))
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got.astype(np.float64) - ref) / max(nref, 1e-30))
    print(f"[bwd] {name}: max-abs {err:.3e} of scale {scale:.3e}, relative norm {rel:.3e}", flush=True)
    assert np.all(np.isfinite(got)), name
    # 1e-4 absolute floor: where the exact gradient vanishes (one token: dP equals Dv), the
    # kernel's two FP32 evaluations of the same 128-term dot product differ by rounding only
    assert err <= 2e-2 * scale + 1e-4, name
    if nref > 1e-6:
        assert rel <= 1e-2, name


@pytest.mark.parametrize("B,Hq,Hkv,S,norm", [
    (2, 8, 2, 70, True),      # ragged tail past two 32-tiles, GQA group 4
    (1, 4, 4, 33, True),      # group 1
    (1, 16, 2, 48, True),     # group 8: each wavefront takes two query heads
    (2, 8, 2, 17, False),     # no RMSNorm on either side
    (1, 4, 1, 1, True),       # one token
])
def test_backward_parity(gpu, B, Hq, Hkv, S, norm):
    (q, k, v, do, wq, wk, pos), res = _run(100 + S, B, Hq, Hkv, S, norm)
    ref = oracle.prefill_forward_backward(q, k, v, wq, wk, pos, do)
    dq, dk, dv, dwq, dwk = res[0]
    _check("dq", dq, ref[2])
    _check("dk", dk, ref[3])
    _check("dv", dv, ref[4])
    if norm:
        _check("dw_q", dwq, ref[5])
        _check("dw_k", dwk, ref[6])
    else:
        assert dwq is None and dwk is None


def test_backward_bitwise_repeatable(gpu):
    _, res = _run(7, 2, 8, 2, 96, True, repeats=3)
    for r in res[1:]:
        for a, b in zip(res[0], r):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_backward_row_alone_equals_row_in_batch(gpu):
    """dq, dk, dv of a row depend only on that row (the weight gradients sum over the batch)."""
    q, k, v, do, wq, wk, pos = _case(9, 3, 8, 2, 50)
    f = lambda a: torch.from_numpy(a).cuda()
    outs = []
    for sel in (slice(0, 3), slice(1, 2)):
        qs, ks, vs, ds, ps = q[sel], k[sel], v[sel], do[sel], pos[sel]
        plan = pa.Plan(8, 2, max_batch=3, max_q_len=50, max_pages_per_row=4)
        out, lse = _forward(plan, qs, ks, vs, wq, wk, ps)
        g = pa.prefill_backward(plan, i32(ps), bf16_tensor(qs), bf16_tensor(ks), bf16_tensor(vs), out, lse,
                                bf16_tensor(ds), q_norm_weight=f(wq), k_norm_weight=f(wk))
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in g[:3]])
    for full, alone in zip(outs[0], outs[1]):
        assert np.array_equal(full[1:2].view(np.uint32), alone.view(np.uint32))


def test_backward_positions_not_in_token_order(gpu):
    """Visibility follows positions, not token order: row 0 holds a permutation of 0..S-1, row 1
    starts at 37.  Tiles are skipped only where every pair is masked, so the gradients still
    match the oracle.  out and lse come from the oracle's forward (the paged forward places
    keys at their token index)."""
    rng = np.random.default_rng(77)
    B, Hq, Hkv, S = 2, 8, 2, 150
    q, k, v, do, wq, wk, _ = _case(78, B, Hq, Hkv, S)
    pos = np.stack([rng.permutation(S), 37 + np.arange(S)]).astype(np.int32)
    ref = oracle.prefill_forward_backward(q, k, v, wq, wk, pos, do)
    out = bf16_tensor(oracle.bf16_bits_from_f32(ref[0].astype(np.float32)))
    lse = torch.from_numpy(ref[1].astype(np.float32)).cuda()
    plan = pa.Plan(Hq, Hkv, max_batch=B, max_q_len=S, max_pages_per_row=16)
    f = lambda a: torch.from_numpy(a).cuda()
    g = pa.prefill_backward(plan, i32(pos), bf16_tensor(q), bf16_tensor(k), bf16_tensor(v), out, lse,
                            bf16_tensor(do), q_norm_weight=f(wq), k_norm_weight=f(wk))
    torch.cuda.synchronize()
    for name, got, r in zip(("dq", "dk", "dv", "dw_q", "dw_k"), g, ref[2:]):
        _check(name, got.cpu().numpy(), r)


def test_backward_out_of_range_position_poisons_its_token(gpu):
    """A token whose position lies outside the RoPE table gets NaN dq and dk rows (its q^ and k^
    are NaN, so whatever they reach in its own row is NaN too); the other row keeps the bits of
    a clean run, since rows never mix."""
    B, Hq, Hkv, S = 2, 8, 2, 40
    q, k, v, do, wq, wk, pos = _case(31, B, Hq, Hkv, S)
    plan = pa.Plan(Hq, Hkv, max_batch=B, max_q_len=S, max_pages_per_row=3)  # RoPE table: 49 rows
    out, lse = _forward(plan, q, k, v, wq, wk, pos)
    f = lambda a: torch.from_numpy(a).cuda()
    res = []
    bad = pos.copy()
    bad[0, 5] = 10_000
    for p in (pos, bad):
        g = pa.prefill_backward(plan, i32(p), bf16_tensor(q), bf16_tensor(k), bf16_tensor(v), out, lse,
                                bf16_tensor(do), q_norm_weight=f(wq), k_norm_weight=f(wk))
        torch.cuda.synchronize()
        res.append([t.cpu().numpy() for t in g[:3]])
    (dq0, dk0, dv0), (dq1, dk1, dv1) = res
    assert np.all(np.isfinite(dq0)) and np.all(np.isfinite(dk0)) and np.all(np.isfinite(dv0))
    assert np.all(np.isnan(dq1[0, :, 5])) and np.all(np.isnan(dk1[0, :, 5]))
    for clean, poisoned in ((dq0, dq1), (dk0, dk1), (dv0, dv1)):
        assert np.array_equal(clean[1].view(np.uint32), poisoned[1].view(np.uint32))


def test_backward_full_size_sampled_group(gpu):
    """The bench's backward launch (B = 4 rows of 2,048 tokens at positions 0..2047, Hq 32 / Hkv 8,
    both norms): every gradient finite, and one row's KV group (4 query heads, 1 KV head) against
    the oracle run on that group alone (a group's dq, dk and dv depend on nothing else)."""
    B, Hq, Hkv, S = 4, 32, 8, 2048
    q, k, v, do, wq, wk, pos = _case(4242, B, Hq, Hkv, S)
    plan = pa.Plan(Hq, Hkv, max_batch=B, max_q_len=S, max_pages_per_row=S // 16)
    out, lse = _forward(plan, q, k, v, wq, wk, pos)
    f = lambda a: torch.from_numpy(a).cuda()
    g = pa.prefill_backward(plan, i32(pos), bf16_tensor(q), bf16_tensor(k), bf16_tensor(v), out, lse,
                            bf16_tensor(do), q_norm_weight=f(wq), k_norm_weight=f(wk))
    torch.cuda.synchronize()
    dq, dk, dv, dwq, dwk = [t.cpu().numpy() for t in g]
    for t in (dq, dk, dv, dwq, dwk):
        assert np.all(np.isfinite(t))
    b, hk = 2, 5
    hq = slice(4 * hk, 4 * hk + 4)
    ref = oracle.prefill_forward_backward(q[b:b + 1, hq], k[b:b + 1, hk:hk + 1], v[b:b + 1, hk:hk + 1], wq, wk,
                                          pos[b:b + 1], do[b:b + 1, hq])
    _check("dq", dq[b:b + 1, hq], ref[2])
    _check("dk", dk[b:b + 1, hk:hk + 1], ref[3])
    _check("dv", dv[b:b + 1, hk:hk + 1], ref[4])
