"""pa_validate_metadata: one negative case per rule, the report's row/index/value, and rule order.

Only the validator sees the broken metadata; no attention kernel is launched on it."""

import numpy as np
import pytest

import deterministic_paged_kv_amd as pa
import workloads
from _paged import i32, make_plan

pytestmark = pytest.mark.gpu


def base_batch():
    # pages per row 3, 1, 2, 6: kv_indptr = [0, 3, 4, 6, 12]
    return workloads.make_batch(21, [40, 3, 17, 96], q_len=3, num_q_heads=8, num_kv_heads=2,
                                num_pages=64, query_mode="prefill")


def decode_batch_with_empty_row():
    # an empty row is only consistent with a single query at position 0
    return workloads.make_batch(22, [40, 0, 17], q_len=1, num_q_heads=8, num_kv_heads=2, num_pages=64)


def validate(b, plan=None, **override):
    plan = plan or make_plan(b, max_pages_per_row=8)
    m = dict(kv_indptr=b.kv_indptr, kv_indices=b.kv_indices, kv_last_page_len=b.kv_last_page_len,
             cache_position=b.cache_position, query_position_ids=b.query_position_ids,
             key_position_ids=b.key_position_ids)
    m.update(override)
    return pa.validate_metadata(plan, batch=b.batch, q_len=b.q_len, num_pages=b.num_pages,
                                **{k: i32(v) for k, v in m.items()})


def test_valid_metadata_passes(gpu):
    b = base_batch()
    assert validate(b)["status"] == "PA_OK"
    d = workloads.tiny_decode()
    assert validate(d, plan=make_plan(d))["status"] == "PA_OK"
    e = decode_batch_with_empty_row()
    assert validate(e)["status"] == "PA_OK"


def test_indptr_rules(gpu):
    b = base_batch()
    x = b.kv_indptr.copy(); x[0] = 1
    rep = validate(b, kv_indptr=x)
    assert rep["status"] == "PA_ERR_INDPTR" and rep["index"] == 0
    x = b.kv_indptr.copy(); x[2] = x[1] - 1
    assert validate(b, kv_indptr=x)["status"] == "PA_ERR_INDPTR"
    x = b.kv_indptr.copy(); x[-1] -= 1
    rep = validate(b, kv_indptr=x)
    assert rep["status"] == "PA_ERR_INDPTR" and rep["index"] == b.batch


def test_capacity_rule(gpu):
    b = base_batch()   # row 3 has 6 pages
    rep = validate(b, plan=make_plan(b, max_pages_per_row=5))
    assert rep["status"] == "PA_ERR_CAPACITY" and rep["row"] == 3 and rep["value"] == 6


def test_page_bounds_rule(gpu):
    b = base_batch()
    x = b.kv_indices.copy(); x[5] = b.num_pages
    rep = validate(b, kv_indices=x)
    assert rep["status"] == "PA_ERR_PAGE_OOB" and rep["index"] == 5 and rep["value"] == b.num_pages
    assert rep["row"] == 2
    x = b.kv_indices.copy(); x[0] = -3
    rep = validate(b, kv_indices=x)
    assert rep["status"] == "PA_ERR_PAGE_OOB" and rep["index"] == 0 and rep["value"] == -3


def test_duplicate_page_rule(gpu):
    b = base_batch()
    x = b.kv_indices.copy(); x[7] = x[1]
    rep = validate(b, kv_indices=x)
    assert rep["status"] == "PA_ERR_DUPLICATE_PAGE" and rep["index"] == 1 and rep["row"] == 0


def test_last_page_len_rules(gpu):
    b = base_batch()
    for bad, row in (([0, 3, 1, 16], 0), ([8, 3, 17, 16], 2)):
        rep = validate(b, kv_last_page_len=np.array(bad))
        assert rep["status"] == "PA_ERR_LAST_PAGE_LEN" and rep["row"] == row, (bad, rep)
    e = decode_batch_with_empty_row()
    rep = validate(e, kv_last_page_len=np.array([8, 2, 1]))   # a row with no pages must say 1
    assert rep["status"] == "PA_ERR_LAST_PAGE_LEN" and rep["row"] == 1, rep


def test_key_position_rule(gpu):
    b = base_batch()
    x = b.key_position_ids.copy()
    base = int(b.kv_indptr[3]) * 16
    x[base + 50] = 49
    rep = validate(b, key_position_ids=x)
    assert rep["status"] == "PA_ERR_KEY_POSITION" and rep["index"] == base + 50 and rep["row"] == 3
    # entries past a row's length are ignored
    x = b.key_position_ids.copy()
    x[int(b.kv_indptr[2]) * 16 + 20] = 12345   # row 2 has 17 keys in 2 pages: slot 20 is past its end
    assert validate(b, key_position_ids=x)["status"] == "PA_OK"


def test_query_position_rules(gpu):
    b = base_batch()
    x = b.query_position_ids.copy(); x[0, 1] += 1               # not contiguous
    rep = validate(b, query_position_ids=x, cache_position=x)
    assert rep["status"] == "PA_ERR_QUERY_POSITION" and rep["row"] == 0
    x = b.query_position_ids.copy(); x[2] -= 1                   # not trailing
    rep = validate(b, query_position_ids=x, cache_position=x)
    assert rep["status"] == "PA_ERR_QUERY_POSITION" and rep["row"] == 2
    x = b.query_position_ids.copy(); x[3] += 1                   # ending at L (decode-style): allowed
    assert validate(b, query_position_ids=x, cache_position=x)["status"] == "PA_OK"


def test_cache_position_rule(gpu):
    b = base_batch()
    x = b.cache_position.copy(); x[3, 2] += 7
    rep = validate(b, cache_position=x)
    assert rep["status"] == "PA_ERR_CACHE_POSITION" and rep["row"] == 3 and rep["index"] == 3 * 3 + 2


def test_first_rule_in_order_is_reported(gpu):
    b = base_batch()
    cp = b.cache_position.copy(); cp[0, 0] += 1
    ind = b.kv_indices.copy(); ind[9] = ind[2]
    rep = validate(b, cache_position=cp, kv_indices=ind)
    assert rep["status"] == "PA_ERR_DUPLICATE_PAGE" and rep["index"] == 2
