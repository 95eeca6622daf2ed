"""pa_decode and pa_prefill captured in a HIP graph (torch.cuda.CUDAGraph drives hipStreamBeginCapture).

The pages ask that graph replay be bitwise equal to eager execution and that no host
synchronisation be needed when the block table changes between calls ("flashinfer_fa2 backend
for NVIDIA Ada (SM89)", "Design notes": CSR metadata built on the device with a fixed shape and
no host synchronisation, graph replay equal to eager; the author's reply to the maintainer
review confirms the replay-vs-eager equality).
The calls read every piece of metadata from device memory and allocate nothing, so a graph
captured once serves any block table of the same shapes.

Each test captures one call, then replays it several times with eager work and host
synchronisations between the replays, poisons the outputs before every replay, and checks
each replay bitwise against an eager call on the same inputs.  Half-way through, new
metadata (other lengths, other pages, other queries, same shapes) is copied into the
captured buffers and the replays must follow it.
"""

import numpy as np
import pytest
import torch

import workloads
import deterministic_paged_kv_amd as pa
from _paged import DeviceBatch, make_plan, same_bits, to_numpy

pytestmark = pytest.mark.gpu

_FIELDS = ("q", "k_cache", "v_cache", "kv_indptr", "kv_indices", "kv_last_page_len", "cache_position",
           "query_position_ids", "key_position_ids", "q_norm_weight", "k_norm_weight")


def _load_into(dst: DeviceBatch, src: DeviceBatch):
    for name in _FIELDS:
        d, s = getattr(dst, name), getattr(src, name)
        assert d.shape == s.shape and d.dtype == s.dtype, name
        d.copy_(s)


def _two_batches(seed, lengths, **kw):
    """Two seeded batches with the same tensor shapes: the second has the row lengths in another
    order (so the same page count), its own page permutation and its own q, K and V."""
    a = workloads.make_batch(seed, lengths, **kw)
    b = workloads.make_batch(seed + 1, list(reversed(lengths)), **kw)
    assert a.nnz == b.nnz
    return a, b


def _replay_and_check(kind, plan, batches, **call_kw):
    fn = pa.decode if kind == "decode" else pa.prefill
    static = DeviceBatch(batches[0])
    out = torch.empty_like(static.q)
    lse = torch.empty(static.q.shape[:3], dtype=torch.float32, device=static.q.device)
    # warm up on a side stream (first launches load the code object), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(plan, *static.args(), out=out, lse=lse, **call_kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn(plan, *static.args(), out=out, lse=lse, **call_kw)
    torch.cuda.synchronize()

    other = DeviceBatch(batches[1])  # eager work between replays uses its own tensors
    eager_ws = {k: (torch.empty_like(v) if v is not None else None) for k, v in call_kw.items()}
    for i, host in enumerate(batches):
        dev = DeviceBatch(host)
        ref = to_numpy(*fn(plan, *dev.args(), **eager_ws))
        if i > 0:
            _load_into(static, dev)
            torch.cuda.synchronize()
        for rep in range(3):
            out.fill_(float("nan"))
            lse.fill_(float("nan"))
            graph.replay()
            fn(plan, *other.args(), **eager_ws)  # unrelated eager call on the same stream
            got = to_numpy(out, lse)
            assert same_bits(got, ref), f"{kind}: replay {rep} of metadata set {i} differs from eager"
            print(f"[graph] {kind} metadata set {i} replay {rep}: bitwise equal to eager", flush=True)
    del graph


def test_decode_graph_replay_one_workgroup_per_unit(gpu):
    a, b = _two_batches(31, [300, 17, 1, 1000, 64], q_len=1, num_q_heads=16, num_kv_heads=4, num_pages=160)
    plan = make_plan(a, max_pages_per_row=64)
    _replay_and_check("decode", plan, (a, b))


def test_decode_graph_replay_multi_cu(gpu):
    a, b = _two_batches(33, [300, 17, 0, 1000, 64], q_len=1, num_q_heads=16, num_kv_heads=4, num_pages=160)
    plan = make_plan(a, max_pages_per_row=64)
    ws = pa.decode_workspace(plan, a.batch)
    _replay_and_check("decode", plan, (a, b), workspace=ws)


def test_prefill_graph_replay(gpu):
    a, b = _two_batches(35, [40, 200, 97, 64], q_len=40, num_q_heads=8, num_kv_heads=2, num_pages=40,
                        query_mode="prefill")
    plan = make_plan(a, max_pages_per_row=16)
    ws = torch.empty(pa.prefill_workspace_size(plan, a.batch, a.q_len, a.nnz), dtype=torch.uint8,
                     device="cuda")
    _replay_and_check("prefill", plan, (a, b), workspace=ws)


def test_decode_plan_width_switches_inside_one_graph(gpu):
    """Plans of width 64, 65 and 128 pages called back to back inside one captured graph (a host
    synchronisation anywhere in the calls would abort the capture), each writing its own out and
    lse.  Every replay, with new metadata copied in between, gives the three results bitwise equal
    to each other and to eager calls: the plan width is capacity only ("flashinfer_fa2 backend
    for NVIDIA Ada (SM89)", "Design notes": plans keyed by a power-of-two width bucket, no host
    synchronisation when the width changes)."""
    a, b = _two_batches(37, [300, 17, 0, 1000, 64], q_len=1, num_q_heads=16, num_kv_heads=4, num_pages=160)
    plans = [make_plan(a, max_pages_per_row=w) for w in (64, 65, 128)]
    static = DeviceBatch(a)
    ws = [pa.decode_workspace(p, a.batch) for p in plans]
    outs = [torch.empty_like(static.q) for _ in plans]
    lses = [torch.empty(static.q.shape[:3], dtype=torch.float32, device="cuda") for _ in plans]

    def calls():
        for i, p in enumerate(plans):
            # the middle plan runs the one-workgroup schedule, the others the multi-CU one
            pa.decode(p, *static.args(), out=outs[i], lse=lses[i], workspace=None if i == 1 else ws[i])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    for i, host in enumerate((a, b)):
        dev = DeviceBatch(host)
        ref = to_numpy(*pa.decode(plans[2], *dev.args()))
        if i > 0:
            _load_into(static, dev)
            torch.cuda.synchronize()
        for rep in range(3):
            for o, l in zip(outs, lses):
                o.fill_(float("nan"))
                l.fill_(float("nan"))
            graph.replay()
            pa.decode(plans[0], *dev.args())  # an eager call of another width between replays
            for w, o, l in zip((64, 65, 128), outs, lses):
                assert same_bits(to_numpy(o, l), ref), f"width {w}, metadata set {i}, replay {rep}"
            print(f"[graph] widths 64/65/128 in one graph, metadata set {i} replay {rep}: bitwise equal", flush=True)
    del graph
