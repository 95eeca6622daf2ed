"""pa_build_csr on the GPU: bit-exact against the CPU reference on thousands of random tables,
and its output driving pa_decode / pa_prefill (also inside a HIP graph).

The pages' audit checked their CSR construction against a reference on 2,000 random cases
with empty rows, -1 table padding and widths 1-40, and asked for an empty row in the
reference test ("flashinfer_fa2 backend for NVIDIA Ada (SM89)", "Code audit").
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
import deterministic_paged_kv_amd as pa
from _paged import DeviceBatch, i32, key_positions_for, make_plan, same_bits, to_numpy

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def _gpu_csr(table, lens):
    indptr, indices, last = pa.build_csr(i32(table), i32(lens))
    torch.cuda.synchronize()
    return indptr.cpu().numpy(), indices.cpu().numpy(), last.cpu().numpy()


def _random_case(rng):
    B = int(rng.integers(1, 10))
    width = int(rng.integers(1, 41))
    lens = rng.integers(0, 16 * width + 1, size=B)
    pick = rng.random(B)
    lens[pick < 0.2] = 0                                   # empty rows
    lens[(pick >= 0.2) & (pick < 0.3)] = 16 * width        # full rows
    edge = (pick >= 0.3) & (pick < 0.4)                    # page boundaries
    lens[edge] = 16 * rng.integers(0, width + 1, size=int(edge.sum()))
    table = rng.integers(0, 100000, size=(B, width)).astype(np.int32)
    for b in range(B):
        table[b, -(-int(lens[b]) // 16):] = -1             # -1 padding past the live pages
    return table, lens.astype(np.int32)


def test_worked_example(gpu):
    g = json.load(open(os.path.join(HERE, "golden", "csr_example.json")))
    got = _gpu_csr(np.array(g["block_table"], dtype=np.int32), np.array(g["kv_lens"], dtype=np.int32))
    assert got[0].tolist() == g["kv_indptr"]
    assert got[1].tolist() == g["kv_indices"]
    assert got[2].tolist() == g["kv_last_page_len"]


def test_random_tables_bit_exact(gpu):
    rng = np.random.default_rng(2024)
    for case in range(2000):
        table, lens = _random_case(rng)
        if case % 50 == 7:                                 # an unrepresentable length now and then
            lens[0] = 16 * table.shape[1] + 1 if case % 100 == 7 else -3
        got = _gpu_csr(table, lens)
        ref = oracle.csr_from_block_table(table, lens)
        for name, a, r in zip(("indptr", "indices", "last_page_len"), got, ref):
            assert np.array_equal(a, r), f"case {case} (B={table.shape[0]}, W={table.shape[1]}): {name}"
    print("[csr] 2000 random tables bit-exact", flush=True)


def test_large_batch_running_sum(gpu):
    """More rows than the running-sum workgroup has threads (1024)."""
    rng = np.random.default_rng(5)
    B, W = 3000, 7
    lens = rng.integers(0, 16 * W + 1, size=B).astype(np.int32)
    table = rng.integers(0, 1 << 20, size=(B, W)).astype(np.int32)
    got = _gpu_csr(table, lens)
    ref = oracle.csr_from_block_table(table, lens)
    for a, r in zip(got, ref):
        assert np.array_equal(a, r)


def _dense_from(batch, width):
    B = batch.batch
    t = np.full((B, width), -1, dtype=np.int32)
    for b in range(B):
        row = batch.kv_indices[batch.kv_indptr[b]:batch.kv_indptr[b + 1]]
        t[b, :len(row)] = row
    return t, batch.lengths.astype(np.int32)


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_device_csr_drives_attention_bitwise(gpu, kind):
    """Attention over the device-built CSR (num_indices = B * width, -1 tail) equals attention
    over the compact host-built CSR of the same rows, bit for bit."""
    if kind == "decode":
        b = workloads.make_batch(41, [300, 0, 17, 1000, 64], q_len=1, num_q_heads=16, num_kv_heads=4,
                                 num_pages=160)
    else:
        b = workloads.make_batch(42, [40, 200, 97, 64], q_len=40, num_q_heads=8, num_kv_heads=2,
                                 num_pages=64, query_mode="prefill")
    width = 64
    plan = make_plan(b, max_pages_per_row=width)
    db = DeviceBatch(b)
    fn = pa.decode if kind == "decode" else pa.prefill
    ref = to_numpy(*fn(plan, *db.args()))
    table, lens = _dense_from(b, width)
    indptr, indices, last = pa.build_csr(i32(table), i32(lens))
    args = list(db.args())
    args[3], args[4], args[5] = indptr, indices, last
    args[8] = key_positions_for(b, int(indices.numel()))
    got = to_numpy(*fn(plan, *args))
    assert same_bits(got, ref), kind
    print(f"[csr] {kind} over the device-built CSR: bitwise equal", flush=True)


def test_unrepresentable_length_fails_loudly(gpu):
    """A row longer than its table gets last_page_len 0: the validator names it and decode
    writes NaN for that row only."""
    b = workloads.make_batch(43, [40, 70], q_len=1, num_q_heads=8, num_kv_heads=2, num_pages=16)
    width = 5
    table, lens = _dense_from(b, width)
    lens[1] = 16 * width + 3
    indptr, indices, last = pa.build_csr(i32(table), i32(lens))
    torch.cuda.synchronize()
    assert last.cpu().tolist() == [8, 0]
    plan = make_plan(b, max_pages_per_row=width)
    db = DeviceBatch(b)
    args = list(db.args())
    args[3], args[4], args[5] = indptr, indices, last
    args[8] = key_positions_for(b, int(indices.numel()))
    out, lse = to_numpy(*pa.decode(plan, *args))
    assert np.all(np.isnan(lse[1])) and np.all(np.isfinite(lse[0]))
    nnz = int(indptr[-1].item())
    rep = pa.validate_metadata(plan, batch=2, q_len=1, num_pages=b.num_pages, kv_indptr=indptr,
                               kv_indices=indices[:nnz].contiguous(), kv_last_page_len=last,
                               cache_position=db.cache_position, query_position_ids=db.query_position_ids,
                               key_position_ids=db.key_position_ids)
    assert nnz == b.nnz
    assert rep["status"] == "PA_ERR_LAST_PAGE_LEN" and rep["row"] == 1, rep


def test_build_and_decode_in_one_graph(gpu):
    """pa_build_csr + pa_decode captured together: replays follow new tables and lengths copied
    into the captured buffers (no host synchronisation anywhere), bitwise equal to eager."""
    width = 64
    kw = dict(q_len=1, num_q_heads=16, num_kv_heads=4, num_pages=160)
    a = workloads.make_batch(51, [300, 17, 0, 1000, 64], **kw)
    c = workloads.make_batch(52, [64, 1000, 5, 17, 300], **kw)
    plan = make_plan(a, max_pages_per_row=width)
    ta, la = _dense_from(a, width)
    static = DeviceBatch(a)
    table, lens = i32(ta), i32(la)
    indptr = torch.empty(a.batch + 1, dtype=torch.int32, device="cuda")
    indices = torch.empty(a.batch * width, dtype=torch.int32, device="cuda")
    last = torch.empty(a.batch, dtype=torch.int32, device="cuda")
    out = torch.empty_like(static.q)
    lse = torch.empty(static.q.shape[:3], dtype=torch.float32, device="cuda")

    kpos = key_positions_for(a, a.batch * width)

    def call():
        pa.build_csr(table, lens, indptr, indices, last)
        args = list(static.args())
        args[3], args[4], args[5], args[8] = indptr, indices, last, kpos
        pa.decode(plan, *args, out=out, lse=lse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for i, host in enumerate((a, c)):
        dev = DeviceBatch(host)
        ref = to_numpy(*pa.decode(plan, *dev.args()))
        t, l = _dense_from(host, width)
        table.copy_(i32(t))
        lens.copy_(i32(l))
        for name in ("q", "k_cache", "v_cache", "cache_position", "query_position_ids", "q_norm_weight",
                     "k_norm_weight"):
            getattr(static, name).copy_(getattr(dev, name))
        kpos.copy_(key_positions_for(host, a.batch * width))
        for rep in range(3):
            out.fill_(float("nan"))
            indices.fill_(12345)
            graph.replay()
            got = to_numpy(out, lse)
            assert same_bits(got, ref), f"table {i} replay {rep}"
    print("[csr] build + decode graph replays bitwise equal to eager", flush=True)
    del graph
