"""The oracle's result on the tiny decode workload is frozen in tests/golden/."""
import hashlib
import json
import os

import numpy as np

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_decode_oracle.json")


def test_oracle_matches_frozen_tiny_decode():
    doc = json.load(open(GOLDEN))
    b = workloads.tiny_decode()
    digest = hashlib.sha256(b.q.tobytes() + b.k_cache.tobytes() + b.v_cache.tobytes()).hexdigest()
    assert digest == doc["inputs_sha256"], "seeded generator changed"
    args, kwargs = b.oracle_args()
    out, lse = oracle.paged_attention(*args, **kwargs)
    np.testing.assert_array_equal(out[:, :, 0, :], np.array(doc["out_bf16_bits"], dtype=np.uint16))
    np.testing.assert_array_equal(lse[:, :, 0], np.array(doc["lse"], dtype=np.float32))
