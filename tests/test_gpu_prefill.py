"""pa_prefill on the GPU against the CPU oracle, and its bitwise invariances."""

import numpy as np
import pytest

import oracle
import workloads
from _paged import DeviceBatch, assert_parity, make_plan, run

pytestmark = pytest.mark.gpu


def oracle_ref(b, rows=None, q_heads=None):
    args, kwargs = b.oracle_args()
    return oracle.paged_attention(*args, rows=rows, q_heads=q_heads, **kwargs)


def test_chunked_prefill_parity(gpu):
    """B=4 x 512-query chunks after prefixes 0/1024/2048/3584, Hq=32, Hkv=8: full oracle."""
    b = workloads.chunked_prefill()
    db = DeviceBatch(b)
    out, lse = run("prefill", make_plan(b), db)
    ref_out, ref_lse = oracle_ref(b)
    assert_parity(out, lse, ref_out, ref_lse, "chunked prefill", kind="prefill")


@pytest.mark.parametrize("lengths,q_len", [
    ([37, 100, 101], 37),          # ragged query block, a row with no prefix
    ([1, 16, 17, 80], 1),          # single query (decode-shaped prefill)
    ([64, 65, 200], 64),
    ([5, 300], 5),
])
def test_prefill_ragged(gpu, lengths, q_len):
    b = workloads.make_batch(31, lengths, q_len=q_len, num_q_heads=8, num_kv_heads=2, num_pages=64,
                             query_mode="prefill")
    out, lse = run("prefill", make_plan(b), DeviceBatch(b))
    ref_out, ref_lse = oracle_ref(b)
    assert_parity(out, lse, ref_out, ref_lse, f"prefill {lengths} Sq={q_len}", kind="prefill")


@pytest.mark.parametrize("hq,hkv", [(2, 2), (6, 2), (24, 2), (32, 2)])
def test_prefill_group_sizes(gpu, hq, hkv):
    b = workloads.make_batch(32, [70, 130], q_len=40, num_q_heads=hq, num_kv_heads=hkv, num_pages=32,
                             query_mode="prefill")
    out, lse = run("prefill", make_plan(b), DeviceBatch(b))
    ref_out, ref_lse = oracle_ref(b)
    assert_parity(out, lse, ref_out, ref_lse, f"prefill Hq={hq} Hkv={hkv}", kind="prefill")


def test_prefill_row_past_the_page_table(gpu):
    """A row of more than 2,048 pages (the attention kernel's LDS page table) looks its pages up
    with scalar loads instead; a short row beside it keeps the table."""
    b = workloads.make_batch(35, [40_000, 300], q_len=32, num_q_heads=8, num_kv_heads=2, num_pages=2600,
                             query_mode="prefill")
    out, lse = run("prefill", make_plan(b), DeviceBatch(b))
    ref_out, ref_lse = oracle_ref(b)
    assert_parity(out, lse, ref_out, ref_lse, "prefill 40,000-key row", kind="prefill")


def test_prefill_more_units_than_the_ranking_holds(gpu):
    """520 rows of one query each: 520 work units, more than the 512 the prologue ranks, so the
    units run in number order."""
    lengths = np.random.default_rng(36).integers(1, 100, size=520)
    b = workloads.make_batch(36, lengths, q_len=1, num_q_heads=8, num_kv_heads=2, num_pages=4096,
                             query_mode="prefill")
    out, lse = run("prefill", make_plan(b), DeviceBatch(b))
    ref_out, ref_lse = oracle_ref(b)
    assert_parity(out, lse, ref_out, ref_lse, "prefill, 520 units", kind="prefill")


def test_prefill_decode_style_positions_and_no_norm(gpu):
    """Queries ending at L (keys of the chunk not all cached), and no RMSNorm."""
    b = workloads.make_batch(33, [50, 90], q_len=8, num_q_heads=8, num_kv_heads=2, num_pages=32,
                             query_mode="decode", norm=False)
    out, lse = run("prefill", make_plan(b), DeviceBatch(b))
    ref_out, ref_lse = oracle_ref(b)
    assert_parity(out, lse, ref_out, ref_lse, "prefill decode-style positions", kind="prefill")


def test_prefill_row_alone_equals_row_in_batch(gpu):
    full = workloads.chunked_prefill(seed=34)
    plan = make_plan(full)
    o_full, l_full = run("prefill", plan, DeviceBatch(full))
    again = run("prefill", plan, DeviceBatch(full))
    assert np.array_equal(o_full, again[0]) and np.array_equal(l_full.view(np.uint32), again[1].view(np.uint32))
    r = 2
    lo, hi = int(full.kv_indptr[r]), int(full.kv_indptr[r + 1])
    alone = workloads.PagedBatch(**{**full.__dict__,
                                    "q": full.q[r:r + 1].copy(),
                                    "kv_indptr": np.array([0, hi - lo], np.int32),
                                    "kv_indices": full.kv_indices[lo:hi].copy(),
                                    "kv_last_page_len": full.kv_last_page_len[r:r + 1].copy(),
                                    "cache_position": full.cache_position[r:r + 1].copy(),
                                    "query_position_ids": full.query_position_ids[r:r + 1].copy(),
                                    "key_position_ids": full.key_position_ids[lo * 16:hi * 16].copy(),
                                    "lengths": full.lengths[r:r + 1].copy()})
    wide = make_plan(alone, max_pages_per_row=1024)
    o_a, l_a = run("prefill", wide, DeviceBatch(alone))
    assert np.array_equal(o_a[0], o_full[r])
    assert np.array_equal(l_a[0].view(np.uint32), l_full[r].view(np.uint32))
    o_p, l_p = run("prefill", wide, DeviceBatch(workloads.permute_pages(alone, 3)))
    assert np.array_equal(o_p[0], o_full[r])
    assert np.array_equal(l_p[0].view(np.uint32), l_full[r].view(np.uint32))


def test_prefill_partial_head_group_ragged_blocks(gpu):
    """Ragged query blocks (Sq = 300), a partial group of query heads (Hq = 24, Hkv = 4, groups of
    4 + 2), rows of different lengths: parity with the oracle, and a row alone bitwise equal to
    the same row in the batch."""
    full = workloads.make_batch(35, [300, 420, 555, 700], q_len=300, num_q_heads=24, num_kv_heads=4,
                                num_pages=256, query_mode="prefill")
    plan = make_plan(full)
    o_full, l_full = run("prefill", plan, DeviceBatch(full))
    ref_out, ref_lse = oracle_ref(full)
    assert_parity(o_full, l_full, ref_out, ref_lse, "prefill, partial head group", kind="prefill")
    r = 1
    lo, hi = int(full.kv_indptr[r]), int(full.kv_indptr[r + 1])
    alone = workloads.PagedBatch(**{**full.__dict__,
                                    "q": full.q[r:r + 1].copy(),
                                    "kv_indptr": np.array([0, hi - lo], np.int32),
                                    "kv_indices": full.kv_indices[lo:hi].copy(),
                                    "kv_last_page_len": full.kv_last_page_len[r:r + 1].copy(),
                                    "cache_position": full.cache_position[r:r + 1].copy(),
                                    "query_position_ids": full.query_position_ids[r:r + 1].copy(),
                                    "key_position_ids": full.key_position_ids[lo * 16:hi * 16].copy(),
                                    "lengths": full.lengths[r:r + 1].copy()})
    o_a, l_a = run("prefill", make_plan(alone, max_pages_per_row=64), DeviceBatch(alone))
    assert np.array_equal(o_a[0], o_full[r])
    assert np.array_equal(l_a[0].view(np.uint32), l_full[r].view(np.uint32))
