"""pa_decode under the fixed-chunk split policy (PA_SPLIT_FIXED, chunks of N tokens folded in
ascending order): oracle parity, and bitwise invariance to the batch, the plan width and the
physical pages ("WS2 PR7 Fused Attention Backend Alignment", "Split-KV Policy": fixed:<N> in
tokens divisible by the page size; "flashinfer_fa2 backend for NVIDIA Ada (SM89)", "Code
audit": a partition that depends only on the row's own length)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
import deterministic_paged_kv_amd as pa
from _paged import DeviceBatch, assert_parity, make_plan, run, same_bits

pytestmark = pytest.mark.gpu


def oracle_ref(b, rows=None, q_heads=None):
    args, kwargs = b.oracle_args()
    return oracle.paged_attention(*args, rows=rows, q_heads=q_heads, **kwargs)


def run_fixed(plan, db, batch):
    ws = pa.decode_workspace(plan, batch)
    ws.fill_(0xFF)  # needs no initialisation
    return run("decode", plan, db, workspace=ws)


@pytest.mark.parametrize("chunk", [16, 32, 128])
def test_tiny_and_ragged_parity(gpu, chunk):
    for label, b in (("tiny", workloads.tiny_decode()),
                     ("ragged", workloads.make_batch(61, [0, 1, 15, 16, 17, 33, 130, 255, 1000], q_len=1,
                                                     num_q_heads=8, num_kv_heads=2, num_pages=256))):
        plan = make_plan(b, chunk_tokens=chunk)
        out, lse = run_fixed(plan, DeviceBatch(b), b.batch)
        ref_out, ref_lse = oracle_ref(b)
        assert_parity(out, lse, ref_out, ref_lse, f"fixed:{chunk} {label}")


@pytest.mark.parametrize("batch,length,chunk", [(1, 131072, 2048)])
def test_long_context_parity_sampled(gpu, batch, length, chunk):
    """The long-context low-batch shape the fixed policy is for (Hq=32, Hkv=8)."""
    b = workloads.long_decode(batch, length, num_pages=batch * length // 16 + 512)
    plan = make_plan(b, max_pages_per_row=length // 16, chunk_tokens=chunk)
    out, lse = run_fixed(plan, DeviceBatch(b), b.batch)
    heads = [0, 5, 31]
    ref_out, ref_lse = oracle_ref(b, rows=[batch - 1], q_heads=heads)
    assert_parity(out[[batch - 1]][:, heads], lse[[batch - 1]][:, heads], ref_out, ref_lse,
                  f"fixed:{chunk} long decode B={batch} L={length}")


def test_batch_width_and_page_invariance(gpu):
    """The 1,500-token row alone under 128- and 256-page plans, as row 3 of a batch of 8 under 512-
    and 1024-page plans, and with its pages permuted: bitwise equal, each repeated."""
    chunk = 256
    alone = workloads.invariance_batch(alone=True)
    full = workloads.invariance_batch(alone=False)
    r = workloads.INVARIANCE_ROW_INDEX
    db_alone, db_full = DeviceBatch(alone), DeviceBatch(full)
    db_perm = DeviceBatch(workloads.permute_pages(alone, 78))
    results = []
    for width in (128, 256):
        plan = make_plan(alone, max_pages_per_row=width, chunk_tokens=chunk)
        for _ in range(5):
            o, l = run_fixed(plan, db_alone, 1)
            results.append((f"alone w={width}", o[0], l[0]))
        o, l = run_fixed(plan, db_perm, 1)
        results.append((f"permuted w={width}", o[0], l[0]))
    for width in (512, 1024):
        plan = make_plan(full, max_pages_per_row=width, max_batch=8, chunk_tokens=chunk)
        for _ in range(5):
            o, l = run_fixed(plan, db_full, 8)
            results.append((f"batch8 w={width}", o[r], l[r]))
    label0, o0, l0 = results[0]
    for label, o, l in results[1:]:
        assert np.array_equal(o, o0), f"out differs: {label} vs {label0}"
        assert np.array_equal(l.view(np.uint32), l0.view(np.uint32)), f"lse differs: {label} vs {label0}"
    ref_out, ref_lse = oracle_ref(alone)
    assert_parity(o0[None], l0[None], ref_out, ref_lse, "fixed:256 1500-token row")
    # a different recorded policy: the bits are not those of the 16-stream tree
    o_dis, l_dis = run("decode", make_plan(alone, max_pages_per_row=128), db_alone)
    assert not (np.array_equal(o_dis[0], o0) and np.array_equal(l_dis[0].view(np.uint32), l0.view(np.uint32)))


def test_policy_errors(gpu):
    b = workloads.tiny_decode()
    plan = make_plan(b, chunk_tokens=64)
    db = DeviceBatch(b)
    with pytest.raises(pa.PagedAttentionError) as e:
        pa.decode(plan, *db.args())            # the fixed policy needs a workspace
    assert e.value.name == "PA_ERR_WORKSPACE"
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(pa.PagedAttentionError) as e:
        pa.decode(plan, *db.args(), workspace=small)
    assert e.value.name == "PA_ERR_WORKSPACE"
    pb = workloads.make_batch(62, [40, 64], q_len=8, num_q_heads=8, num_kv_heads=2, num_pages=16,
                              query_mode="prefill")
    pplan = make_plan(pb, chunk_tokens=64)
    with pytest.raises(pa.PagedAttentionError) as e:
        pa.prefill(pplan, *DeviceBatch(pb).args())
    assert e.value.name == "PA_ERR_UNSUPPORTED"


def test_most_chunks_per_row(gpu):
    """4,096 one-page chunks in one row (the fold's limit): oracle parity on a few heads."""
    b = workloads.make_batch(64, [4096 * 16], q_len=1, num_q_heads=8, num_kv_heads=2, num_pages=4096)
    plan = make_plan(b, max_pages_per_row=4096, chunk_tokens=16)
    out, lse = run_fixed(plan, DeviceBatch(b), b.batch)
    heads = [0, 5]
    ref_out, ref_lse = oracle_ref(b, q_heads=heads)
    assert_parity(out[:, heads], lse[:, heads], ref_out, ref_lse, "fixed:16 with 4,096 chunks")
