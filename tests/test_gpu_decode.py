"""pa_decode on the GPU against the CPU oracle, and its bitwise invariances."""

import functools

import numpy as np
import pytest

import oracle
import workloads
import deterministic_paged_kv_amd as pa
from _paged import DeviceBatch, assert_parity, make_plan, run, same_bits

pytestmark = pytest.mark.gpu


def oracle_ref(b, rows=None, q_heads=None):
    args, kwargs = b.oracle_args()
    return oracle.paged_attention(*args, rows=rows, q_heads=q_heads, **kwargs)


def check_full(b, label, plan=None):
    db = DeviceBatch(b)
    plan = plan or make_plan(b)
    out, lse = run("decode", plan, db)
    ref_out, ref_lse = oracle_ref(b)
    assert_parity(out, lse, ref_out, ref_lse, label)
    return out, lse


def test_tiny_decode_parity(gpu):
    """B=2, Hq=8, Hkv=2, 128 keys per row, pages drawn from a 64-page pool; NaN canaries elsewhere."""
    check_full(workloads.tiny_decode(), "tiny decode")


@functools.lru_cache(maxsize=1)
def _qwen3_8b():
    """The Qwen3-8B per-GPU batch and its oracle result over every row and head (computed once)."""
    b = workloads.qwen3_8b_decode()
    return b, oracle_ref(b)


@pytest.mark.parametrize("schedule", ["unit", "multi_cu", "fixed_1024"])
def test_qwen3_8b_decode_parity_full(gpu, schedule):
    """Full Qwen3-8B per-GPU shape (B=32, Hq=16, Hkv=4, L ~ U[512, 4096]) against the oracle on
    every row and query head.  Three schedules: one workgroup per (row, KV head), the multi-CU
    one (stream kernel + combine, the launch configuration the benchmark times), and the
    fixed-chunk policy with 1,024-token chunks."""
    b, (ref_out, ref_lse) = _qwen3_8b()
    db = DeviceBatch(b)
    plan = make_plan(b, max_pages_per_row=256, chunk_tokens=1024 if schedule == "fixed_1024" else 0)
    ws = pa.decode_workspace(plan, b.batch) if schedule != "unit" else None
    out, lse = run("decode", plan, db, workspace=ws)
    assert_parity(out, lse, ref_out, ref_lse, f"qwen3-8b decode ({schedule}), all 32 rows x 16 heads")


@pytest.mark.parametrize("lengths", [
    [0, 1, 15, 16, 17, 33, 130, 255],
    [2, 0, 0, 31],
    [4096, 3],
])
def test_decode_ragged_and_empty_rows(gpu, lengths):
    b = workloads.make_batch(11, lengths, q_len=1, num_q_heads=8, num_kv_heads=2,
                             num_pages=max(64, 2 * sum((L + 15) // 16 for L in lengths)))
    check_full(b, f"ragged {lengths}")


@pytest.mark.parametrize("hq,hkv", [(4, 4), (6, 2), (16, 2), (32, 2), (32, 8)])
def test_decode_group_sizes(gpu, hq, hkv):
    b = workloads.make_batch(12, [77, 300, 16], q_len=1, num_q_heads=hq, num_kv_heads=hkv, num_pages=128)
    check_full(b, f"Hq={hq} Hkv={hkv}")


def test_decode_without_norm(gpu):
    b = workloads.make_batch(13, [100, 257], q_len=1, num_q_heads=8, num_kv_heads=2, num_pages=64, norm=False)
    check_full(b, "no RMSNorm")


def test_decode_query_at_last_key(gpu):
    """Query position L-1 (the query's own key is the last cached key)."""
    b = workloads.make_batch(14, [50, 129, 1], q_len=1, num_q_heads=8, num_kv_heads=2, num_pages=64)
    b.query_position_ids[:] = (b.lengths - 1)[:, None]
    b.cache_position[:] = b.query_position_ids
    check_full(b, "query at L-1")


def test_decode_bitwise_repeat_and_page_permutation(gpu):
    b = workloads.make_batch(15, [700, 1500, 33, 2048], q_len=1, num_q_heads=16, num_kv_heads=4, num_pages=512)
    plan = make_plan(b)
    db = DeviceBatch(b)
    first = run("decode", plan, db)
    for _ in range(5):
        again = run("decode", plan, db)
        assert np.array_equal(first[0], again[0]) and np.array_equal(first[1].view(np.uint32), again[1].view(np.uint32))
    perm = run("decode", plan, DeviceBatch(workloads.permute_pages(b, 5)))
    assert np.array_equal(first[0], perm[0])
    assert np.array_equal(first[1].view(np.uint32), perm[1].view(np.uint32))


def test_batch_and_plan_width_invariance(gpu):
    """The 1,500-token row (Hq=32, Hkv=8): alone under 128- and 256-page plans, as row 3 of a batch of
    8 under 512- and 1024-page plans, and alone with its pages permuted, through both schedules
    (one workgroup per unit; stream kernel + combine): bitwise equal out and LSE, each run
    repeated; and within tolerance of the oracle."""
    alone = workloads.invariance_batch(alone=True)
    full = workloads.invariance_batch(alone=False)
    r = workloads.INVARIANCE_ROW_INDEX
    results = []
    db_alone = DeviceBatch(alone)
    db_full = DeviceBatch(full)
    db_perm = DeviceBatch(workloads.permute_pages(alone, 77))
    for width in (128, 256):
        plan = make_plan(alone, max_pages_per_row=width)
        for _ in range(10):
            o, l = run("decode", plan, db_alone)
            results.append((f"alone w={width}", o[0], l[0]))
        for _ in range(2):
            o, l = run("decode", plan, db_perm)
            results.append((f"permuted w={width}", o[0], l[0]))
    for width in (512, 1024):
        plan = make_plan(full, max_pages_per_row=width, max_batch=8)
        for _ in range(10):
            o, l = run("decode", plan, db_full)
            results.append((f"batch8 w={width}", o[r], l[r]))
    # the same row through the multi-CU schedule (stream kernel + combine)
    for width in (128, 256):
        plan = make_plan(alone, max_pages_per_row=width)
        ws = pa.decode_workspace(plan, 1)
        for _ in range(3):
            o, l = run("decode", plan, db_alone, workspace=ws)
            results.append((f"alone multi-CU w={width}", o[0], l[0]))
    for width in (512, 1024):
        plan = make_plan(full, max_pages_per_row=width, max_batch=8)
        ws = pa.decode_workspace(plan, 8)
        for _ in range(3):
            o, l = run("decode", plan, db_full, workspace=ws)
            results.append((f"batch8 multi-CU w={width}", o[r], l[r]))
    ref_label, ref_o, ref_l = results[0]
    for label, o, l in results[1:]:
        assert np.array_equal(o, ref_o), f"out differs: {label} vs {ref_label}"
        assert np.array_equal(l.view(np.uint32), ref_l.view(np.uint32)), f"lse differs: {label} vs {ref_label}"
    ref_out, ref_lse = oracle_ref(alone)
    assert_parity(ref_o[None], ref_l[None], ref_out, ref_lse, "1500-token row")


@functools.lru_cache(maxsize=1)
def _long(batch, length):
    return workloads.long_decode(batch, length, num_pages=batch * length // 16 + 512)


@pytest.mark.parametrize("batch,length", [(b, L) for b in (1, 2, 4) for L in (32768, 65536, 131072)])
def test_long_context_grid_parity_all_heads(gpu, batch, length):
    """Every point of the long-context grid the benchmark times (B in {1, 2, 4} x L in {32K, 64K,
    128K}, Hq=32, Hkv=8), under both policies it times (the 16-stream tree on the multi-CU
    schedule, and fixed 1,024-token chunks): all 32 query heads of the batch's last row against
    the oracle."""
    b = _long(batch, length)
    db = DeviceBatch(b)
    ref_out, ref_lse = oracle_ref(b, rows=[batch - 1])
    for chunk in (0, 1024):
        plan = make_plan(b, max_pages_per_row=length // 16, chunk_tokens=chunk)
        ws = pa.decode_workspace(plan, batch)
        out, lse = run("decode", plan, db, workspace=ws)
        policy = f"fixed:{chunk}" if chunk else "tree"
        assert_parity(out[[batch - 1]], lse[[batch - 1]], ref_out, ref_lse,
                      f"long decode B={batch} L={length} ({policy}), all heads of row {batch - 1}")
    del db


@pytest.mark.parametrize("batch,length,schedule", [(1, 131072, "unit"), (2, 32768, "unit")])
def test_long_context_decode_sampled(gpu, batch, length, schedule):
    """Long-context low-batch decode (Hq=32, Hkv=8) on the one-workgroup schedule: oracle on one
    row and two heads per KV group edge."""
    b = _long(batch, length)
    db = DeviceBatch(b)
    plan = make_plan(b, max_pages_per_row=length // 16)
    ws = pa.decode_workspace(plan, batch) if schedule == "multi_cu" else None
    out, lse = run("decode", plan, db, workspace=ws)
    heads = [0, 3, 31]
    ref_out, ref_lse = oracle_ref(b, rows=[batch - 1], q_heads=heads)
    assert_parity(out[[batch - 1]][:, heads], lse[[batch - 1]][:, heads], ref_out, ref_lse,
                  f"long decode B={batch} L={length} ({schedule})")


@pytest.mark.parametrize("name", ["tiny", "ragged", "qwen3_8b", "batch8", "groups16", "kv1", "kv3", "kv6",
                                  "kv3x8", "rows80"])
def test_multi_cu_schedule_is_bit_identical(gpu, name):
    """One wavefront per stream on separate compute units, then a combining kernel, gives the
    same bits as one workgroup per (row, KV head); the workspace needs no initialisation (it is
    filled with NaN bytes before every call)."""
    if name == "tiny":
        b = workloads.tiny_decode()
    elif name == "ragged":
        b = workloads.make_batch(41, [0, 1, 15, 16, 17, 33, 130, 255], q_len=1, num_q_heads=8, num_kv_heads=2,
                                 num_pages=128)
    elif name == "qwen3_8b":
        b = workloads.qwen3_8b_decode()
    elif name == "batch8":
        b = workloads.invariance_batch(alone=False)
    elif name == "groups16":
        b = workloads.make_batch(42, [900, 77], q_len=1, num_q_heads=32, num_kv_heads=2, num_pages=128)
    elif name == "kv3x8":  # 384 single-wavefront workgroups: one dispatch round, second one mirrored
        b = workloads.make_batch(44, [530, 17, 0, 64, 300, 1, 900, 33], q_len=1, num_q_heads=6, num_kv_heads=3,
                                 num_pages=256)
    elif name == "rows80":  # more than 64 rows: launched in row order, no ranking
        lengths = list(np.random.default_rng(45).integers(0, 300, 80))
        b = workloads.make_batch(45, lengths, q_len=1, num_q_heads=8, num_kv_heads=2, num_pages=2048)
    else:  # KV head counts that take one (kv1, kv3) and two (kv6: 12 rows, 1,152 streams) KV heads
        # per workgroup of the multi-CU schedule
        hkv = int(name[2:])
        lengths = [530, 17, 0, 64] * (3 if hkv == 6 else 1)
        b = workloads.make_batch(43, lengths, q_len=1, num_q_heads=2 * hkv, num_kv_heads=hkv, num_pages=256)
    plan = make_plan(b, max_pages_per_row=max(256, int(np.max(np.diff(b.kv_indptr)))))
    db = DeviceBatch(b)
    unit = run("decode", plan, db)
    ws = pa.decode_workspace(plan, b.batch)
    for _ in range(3):
        ws.fill_(0xFF)
        multi = run("decode", plan, db, workspace=ws)
        assert same_bits(unit, multi), name


def test_decode_more_than_64_rows(gpu):
    """80 rows (beyond the on-device ranking's 64) through the multi-CU schedule: oracle parity
    on sampled rows."""
    lengths = list(np.random.default_rng(46).integers(0, 600, 80))
    b = workloads.make_batch(46, lengths, q_len=1, num_q_heads=8, num_kv_heads=2, num_pages=4096)
    plan = make_plan(b)
    ws = pa.decode_workspace(plan, b.batch)
    out, lse = run("decode", plan, DeviceBatch(b), workspace=ws)
    rows = [0, 17, 40, 63, 64, 79]
    ref_out, ref_lse = oracle_ref(b, rows=rows)
    assert_parity(out[rows], lse[rows], ref_out, ref_lse, f"80-row decode rows {rows}")
