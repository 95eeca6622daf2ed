"""Pins of the CSR reference (oracle/csr.py) against a hand-worked example and against the
seeded workload generator, which builds its CSR from lengths by an independent route."""

import json
import os

import numpy as np

import oracle
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


def test_worked_example():
    g = json.load(open(os.path.join(HERE, "golden", "csr_example.json")))
    indptr, indices, last = oracle.csr_from_block_table(np.array(g["block_table"]), np.array(g["kv_lens"]))
    assert indptr.tolist() == g["kv_indptr"]
    assert indices.tolist() == g["kv_indices"]
    assert last.tolist() == g["kv_last_page_len"]


def _dense(indptr, indices, width):
    """The -1-padded dense table of a CSR one."""
    B = len(indptr) - 1
    t = np.full((B, width), -1, dtype=np.int32)
    for b in range(B):
        row = indices[indptr[b]:indptr[b + 1]]
        t[b, :len(row)] = row
    return t


def test_round_trip_with_the_workload_generator():
    rng = np.random.default_rng(7)
    for case in range(300):
        B = int(rng.integers(1, 9))
        width = int(rng.integers(1, 41))
        lens = rng.integers(0, 16 * width + 1, size=B)
        lens[rng.random(B) < 0.2] = 0                          # empty rows
        full = rng.random(B) < 0.1
        lens[full] = 16 * width                                # full rows
        order = rng.permutation(B * width + 7).astype(np.int32)
        indptr, indices, last, _ = workloads.csr_from_lengths(lens, order)
        table = _dense(indptr, indices, width)
        o_indptr, o_indices, o_last = oracle.csr_from_block_table(table, lens)
        nnz = int(indptr[-1])
        assert np.array_equal(o_indptr, indptr), case
        assert np.array_equal(o_indices[:nnz], indices), case
        assert np.all(o_indices[nnz:] == -1), case
        assert np.array_equal(o_last, last), case
