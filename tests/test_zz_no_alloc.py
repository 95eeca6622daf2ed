"""pa_decode_no_alloc (the multi-compute-unit decode with the library's scratch array, for
callers that cannot allocate) against pa_decode with a caller workspace, through the C ABI:
bitwise equal results on two calls in a row, the second with a smaller batch, under both split
policies; and a batch whose workspace exceeds the scratch is rejected before any launch."""

import numpy as np
import pytest
import torch

import workloads
import deterministic_paged_kv_amd as pa
from _paged import DeviceBatch, make_plan, same_bits, to_numpy

pytestmark = pytest.mark.gpu


def _outputs(db):
    return torch.empty_like(db.q), torch.empty(db.q.shape[:3], dtype=torch.float32, device=db.q.device)


@pytest.mark.parametrize("chunk", [0, 256])
def test_no_alloc_decode_matches_workspace_decode(gpu, chunk):
    big = workloads.qwen3_8b_decode()
    small = workloads.make_batch(71, [700, 0, 33, 4096, 1], q_len=1, num_q_heads=16, num_kv_heads=4,
                                 num_pages=1024)
    plan = make_plan(big, max_pages_per_row=256, chunk_tokens=chunk)
    for label, b in (("Qwen3-8B batch", big), ("smaller batch", small)):
        db = DeviceBatch(b)
        ws = pa.decode_workspace(plan, b.batch)
        ref = to_numpy(*pa.decode(plan, *db.args(), workspace=ws))
        out, lse = _outputs(db)
        out.fill_(float("nan"))
        got = to_numpy(*pa.decode_no_alloc(plan, *db.args(), out=out, lse=lse))
        assert same_bits(got, ref), f"{label}, chunk {chunk}"
        assert np.all(np.isfinite(got[1][b.lengths > 0])), label
        print(f"[no-alloc] {label} (chunk {chunk}): bitwise equal to the workspace call", flush=True)


def test_no_alloc_decode_rejects_a_batch_beyond_the_scratch(gpu):
    """126 rows of Hq=16, Hkv=4 need a 16.8 MB workspace, more than the 16 MiB scratch."""
    b = workloads.make_batch(72, [20] * 126, q_len=1, num_q_heads=16, num_kv_heads=4, num_pages=512)
    plan = make_plan(b, max_pages_per_row=4)
    assert pa.decode_workspace_size(plan, 126) > 16 << 20
    db = DeviceBatch(b)
    out, lse = _outputs(db)
    with pytest.raises(pa.PagedAttentionError) as e:
        pa.decode_no_alloc(plan, *db.args(), out=out, lse=lse)
    assert e.value.name == "PA_ERR_CAPACITY"
    small = workloads.make_batch(72, [20] * 125, q_len=1, num_q_heads=16, num_kv_heads=4, num_pages=512)
    assert pa.decode_workspace_size(plan, 125) <= 16 << 20
    sdb = DeviceBatch(small)
    ref = to_numpy(*pa.decode(plan, *sdb.args(), workspace=pa.decode_workspace(plan, 125)))
    out, lse = _outputs(sdb)
    assert same_bits(to_numpy(*pa.decode_no_alloc(plan, *sdb.args(), out=out, lse=lse)), ref)
