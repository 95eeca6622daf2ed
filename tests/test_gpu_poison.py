"""Out-of-range metadata reaching the kernels without validation: the row it belongs to comes out
as NaN (out and LSE), every other row is bitwise what a clean call gives, and nothing is read
out of bounds.

The pages ask that an unsupported or inconsistent request fail closed instead of falling back
or producing a plausible number ("WS2 Attention Cross-Configuration Integration", "Fail closed,
never substitute"; "WS2 PR7 Fused Attention Backend Alignment", "Current Implementation":
metadata checked before execution).  pa_validate_metadata names the violated rule; these tests
cover the calls that run without it.  Every corruption here is one the kernels check before
any access that depends on it (page index against the pool, row extent against the index
array and the plan, last_page_len, query position against the RoPE table).
"""

import numpy as np
import pytest

import workloads
import deterministic_paged_kv_amd as pa
from _paged import DeviceBatch, make_plan, run

pytestmark = pytest.mark.gpu


def _corrupt(db, field, index, value):
    t = getattr(db, field).clone()
    t.view(-1)[index] = value
    setattr(db, field, t)


def _check(clean, bad, bad_row, label):
    out_c, lse_c = clean
    out_b, lse_b = bad
    o = (out_b[bad_row].astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isnan(o)), f"{label}: row {bad_row} out not all NaN"
    assert np.all(np.isnan(lse_b[bad_row])), f"{label}: row {bad_row} lse not all NaN"
    for r in range(out_c.shape[0]):
        if r == bad_row:
            continue
        assert np.array_equal(out_b[r], out_c[r]), f"{label}: row {r} out changed"
        assert np.array_equal(lse_b[r].view(np.uint32), lse_c[r].view(np.uint32)), f"{label}: row {r} lse changed"


def _cases(b, table_rows):
    """(label, field, flat index, value, row it breaks)."""
    ip = b.kv_indptr
    return [
        ("page index past the pool", "kv_indices", int(ip[1]) + 1, b.num_pages + 5, 1),
        ("negative page index", "kv_indices", int(ip[1]) + 2, -2, 1),
        ("last_page_len 17", "kv_last_page_len", 2, 17, 2),
        ("last_page_len 0", "kv_last_page_len", 2, 0, 2),
        ("indptr past the index array", "kv_indptr", 3, int(ip[3]) + 1, 2),
        ("query position past the RoPE table", "query_position_ids", 0, table_rows, 0),
        ("negative query position", "query_position_ids", 0, -1, 0),
        ("cache position not the query position", "cache_position", 0, int(b.query_position_ids[0, -1]) + 3, 0),
        ("key position not the logical index", "key_position_ids", int(ip[1]) * 16 + 7, 8, 1),
    ]


@pytest.mark.parametrize("schedule", ["unit", "multi_cu", "fixed_32"])
def test_decode_out_of_range_metadata_poisons_its_row(gpu, schedule):
    b = workloads.make_batch(61, [40, 100, 70], q_len=1, num_q_heads=8, num_kv_heads=2, num_pages=64)
    plan = make_plan(b, chunk_tokens=32 if schedule == "fixed_32" else 0)
    ws = pa.decode_workspace(plan, b.batch) if schedule != "unit" else None
    clean = run("decode", plan, DeviceBatch(b), workspace=ws)
    table_rows = plan.max_pages_per_row * 16 + 1
    for label, field, idx, value, row in _cases(b, table_rows):
        print(f"[poison] decode {schedule}: {label}", flush=True)
        db = DeviceBatch(b)
        _corrupt(db, field, idx, value)
        _check(clean, run("decode", plan, db, workspace=ws), row, f"decode {schedule}, {label}")


def test_prefill_out_of_range_metadata_poisons_its_row(gpu):
    """One 20-query block per row, so every corruption reaches the whole row."""
    b = workloads.make_batch(62, [50, 90, 33], q_len=20, num_q_heads=8, num_kv_heads=2, num_pages=64,
                             query_mode="prefill")
    plan = make_plan(b)
    clean = run("prefill", plan, DeviceBatch(b))
    table_rows = plan.max_pages_per_row * 16 + 1
    for label, field, idx, value, row in _cases(b, table_rows):
        print(f"[poison] prefill: {label}", flush=True)
        if field in ("query_position_ids", "cache_position"):
            idx = 5  # query 5 of row 0 (every query of the row sees key 7 of row 1)
        db = DeviceBatch(b)
        _corrupt(db, field, idx, value)
        _check(clean, run("prefill", plan, db), row, f"prefill, {label}")


def test_prefill_non_monotone_indptr_poisons_every_row_after_the_decrease(gpu):
    """indptr that decreases after row 0: row 1's extent is negative and row 2's lies inside
    row 0's, so two rows would write k^ into the same workspace rows.  Every row from the
    decrease on comes out NaN; row 0 is bitwise what a clean call gives."""
    b = workloads.make_batch(63, [64, 48, 40, 33], q_len=20, num_q_heads=8, num_kv_heads=2, num_pages=64,
                             query_mode="prefill")
    plan = make_plan(b, max_pages_per_row=16)  # row 2's broken extent (9 pages) fits the plan
    clean = run("prefill", plan, DeviceBatch(b))
    db = DeviceBatch(b)
    _corrupt(db, "kv_indptr", 2, 1)  # [0, 4, 1, ...]: row 1 = [4, 1), row 2 = [1, ...)
    out, lse = run("prefill", plan, db)
    assert np.array_equal(out[0], clean[0][0]) and np.array_equal(lse[0].view(np.uint32), clean[1][0].view(np.uint32))
    for r in range(1, b.batch):
        assert np.all(np.isnan((out[r].astype(np.uint32) << 16).view(np.float32))), f"row {r} out"
        assert np.all(np.isnan(lse[r])), f"row {r} lse"


def test_prefill_bad_page_past_a_block_leaves_that_block_clean(gpu):
    """A page that only later queries see: the queries whose visible keys end before it are
    bitwise unchanged (no NaN from tiles loaded ahead and thrown away), the queries that see it
    are NaN.  One row of 256 new tokens (no prefix), the last page (keys 240..255) out of the
    pool: queries 0..191 lie in blocks that end before key 240 for any block of 32 or 64
    queries."""
    b = workloads.make_batch(64, [256], q_len=256, num_q_heads=8, num_kv_heads=2, num_pages=32,
                             query_mode="prefill")
    plan = make_plan(b)
    clean = run("prefill", plan, DeviceBatch(b))
    db = DeviceBatch(b)
    _corrupt(db, "kv_indices", 15, b.num_pages + 3)
    out, lse = run("prefill", plan, db)
    assert np.array_equal(out[0, :, :192], clean[0][0, :, :192])
    assert np.array_equal(lse[0, :, :192].view(np.uint32), clean[1][0, :, :192].view(np.uint32))
    assert np.all(np.isnan(lse[0, :, 240:]))
    assert np.all(np.isnan((out[0, :, 240:].astype(np.uint32) << 16).view(np.float32)))
