"""Benchmark: paged decode KV GB/s (and chunked prefill TFLOP/s) on one MI355X.

A step is one pa_decode call over the Qwen3-8B per-GPU decode batch: B=32 rows, Hq=16,
Hkv=4, head_dim 128, page 16, kv lengths U{512..4096}, pages scattered over a 16,384-page
pool, bf16 K/V, fused Q/K RMSNorm + RoPE (theta 1e6).  The call is given a workspace, so it
runs the multi-compute-unit schedule (one wavefront per page stream, then a combining
kernel); the schedule without a workspace (one workgroup per row and KV head, bit-identical
results) is timed alongside.  Steps cycle over four independent
K/V pools (same lengths, different pages and contents) so that consecutive steps never find
their K/V in the 256 MB Infinity Cache: each step streams its K/V from HBM.

Printed (one JSON line): value = algorithmic bytes per step / time per step, where the
algorithmic bytes are the K and V bytes of every cached key of every KV head plus q, out,
lse and the CSR metadata the kernel reads (the RoPE table and norm weights are constants
served from cache and are not counted).  The roofline entry divides the same bytes by the
decode call's average time from one pair of HIP events recorded on the launch stream around
the timed calls.
The chunked-prefill workload (B=4 x 512-query chunks after prefixes 0/1024/2048/3584,
Hq=32, Hkv=8) is reported alongside with its algorithmic FLOPs (QK^T and PV over the
causally visible pairs) per call.  The full-prefill backward
(B=4 rows of 2,048 tokens, Hq=32, Hkv=8, Q/K RMSNorm + RoPE) is reported with its algorithmic
FLOPs (five products over the causal pairs).  The CPU oracle is timed on a bounded sample on
the host.

Usage: python bench.py [--gpus 1] [--steps 2000] [--warmup 2000]
       python bench.py --profile-copy     # plain copy of a known size, for counter scaling
       python bench.py --ingest-counters FETCH.csv WRITE.csv COPY_FETCH.csv COPY_WRITE.csv
       python bench.py --ingest-prefill-counters SQ1.csv SQ2.csv FETCH.csv WRITE.csv COPY_FETCH.csv COPY_WRITE.csv
           # rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE results of the decode run and of the copy
           # -> profiles/decode_qwen3_8b_counters.json (HBM bytes per decode launch)
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 MFMA, published (256 CU x 4096 flop/clk x 2.4 GHz)
METRIC = "paged decode KV GB/s (% HBM peak); paged prefill TFLOP/s (% MFMA peak)"
ROTATIONS = 4
PREFILL_ROTATIONS = 8
# untimed calls before each secondary workload (long-context decode, prefill, backward)
SETTLE_MS = 60.0
PREFILL_KERNELS = "prologue_kernel + attend_kernel"


def decode_bytes(b) -> int:
    import numpy as np

    D = 128
    kv = int(np.sum(b.lengths)) * b.num_kv_heads * D * 2 * 2
    q_out = 2 * b.batch * b.num_q_heads * D * 2
    lse = b.batch * b.num_q_heads * 4
    meta = 4 * ((b.batch + 1) + b.nnz + b.batch + b.batch)
    return kv + q_out + lse + meta


def prefill_flops(b) -> int:
    """4 * D * Hq * sum over queries of visible keys (QK^T and PV, causal pairs only)."""
    import numpy as np

    total = 0
    for r in range(b.batch):
        L = int(b.lengths[r])
        pos = b.query_position_ids[r].astype(np.int64)
        total += int(np.sum(np.minimum(pos + 1, L)))
    return 4 * 128 * b.num_q_heads * total


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


DECODE_SOURCES = ["deterministic_paged_kv_amd/csrc/pa_decode.hip", "deterministic_paged_kv_amd/csrc/pa_internal.h"]
PREFILL_SOURCES = ["deterministic_paged_kv_amd/csrc/pa_prefill.hip", "deterministic_paged_kv_amd/csrc/pa_internal.h",
                   "deterministic_paged_kv_amd/csrc/pa_lds_dma.h"]
PREFILL_COUNTERS = os.path.join(ROOT, "profiles", "prefill_chunked_counters.json")


def traffic_from_profile(per_launch_alg_bytes):
    """HBM bytes per decode launch from the committed counter summary, if it matches the source."""
    path = os.path.join(ROOT, "profiles", "decode_qwen3_8b_counters.json")
    if not os.path.exists(path):
        return None
    doc = json.load(open(path))
    if doc.get("source_hash") != source_hash(DECODE_SOURCES):
        return None
    return doc.get("hbm_bytes_per_launch")


def prefill_counters_from_profile():
    """The committed counter summary of the chunked-prefill kernels, if it matches the source."""
    if not os.path.exists(PREFILL_COUNTERS):
        return None
    doc = json.load(open(PREFILL_COUNTERS))
    return doc if doc.get("source_hash") == source_hash(PREFILL_SOURCES) else None


def device_rotation(base, i, device):
    """Pool i of the rotation: the same lengths, a different page permutation and fresh K/V drawn
    on the device (seeded), so the bytes differ from every other pool."""
    import numpy as np
    import torch

    import workloads
    from tests._paged import DeviceBatch

    if i == 0:
        return DeviceBatch(base, device)
    rng = np.random.Generator(np.random.PCG64(5000 + i))
    order = rng.permutation(base.num_pages).astype(np.int32)
    indptr, indices, last, keypos = workloads.csr_from_lengths(base.lengths, order)
    db = DeviceBatch.__new__(DeviceBatch)
    db.host = None
    gen = torch.Generator(device=device)
    gen.manual_seed(7000 + i)
    shape = base.k_cache.shape
    db.k_cache = torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    db.v_cache = torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    db.q = torch.randn(base.q.shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
    db.kv_indptr, db.kv_indices, db.kv_last_page_len = t(indptr), t(indices), t(last)
    db.query_position_ids = t(base.query_position_ids)
    db.cache_position = t(base.cache_position)
    db.key_position_ids = t(keypos)
    db.q_norm_weight = torch.from_numpy(base.q_norm_weight).to(device)
    db.k_norm_weight = torch.from_numpy(base.k_norm_weight).to(device)
    return db


LONG_POOL_PAGES = 40960


def long_context_pool(device, seed=1004):
    """The 40,960-page K/V pool of the long-context decode shape (Hkv=8), drawn on the device."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    shape = (LONG_POOL_PAGES, 16, 8, 128)
    k = torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    return k, v


def long_context_set(batch, length, device, seed=1004, pool=None):
    """The long-context low-batch decode shape (Hq=32, Hkv=8, pages scattered over a 40,960-page
    pool) with K/V/q drawn on the device (seeded); returns (host metadata, device batch).
    `pool` = (k_cache, v_cache) from long_context_pool reuses that pool's K/V."""
    import types

    import numpy as np
    import torch

    import workloads
    from tests._paged import DeviceBatch

    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = np.full(batch, length, dtype=np.int64)
    order = rng.permutation(LONG_POOL_PAGES).astype(np.int32)
    indptr, indices, last, keypos = workloads.csr_from_lengths(lengths, order)
    meta = types.SimpleNamespace(lengths=lengths, num_kv_heads=8, num_q_heads=32, batch=batch,
                                 nnz=int(indptr[-1]))
    db = DeviceBatch.__new__(DeviceBatch)
    db.host = None
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 1)
    db.k_cache, db.v_cache = pool if pool is not None else long_context_pool(device, seed)
    db.q = torch.randn((batch, 32, 1, 128), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
    db.kv_indptr, db.kv_indices, db.kv_last_page_len = t(indptr), t(indices), t(last)
    db.query_position_ids = t(lengths.reshape(batch, 1))
    db.cache_position = db.query_position_ids
    db.key_position_ids = t(keypos)
    db.q_norm_weight = torch.from_numpy(rng.uniform(0.5, 1.5, 128).astype(np.float32)).to(device)
    db.k_norm_weight = torch.from_numpy(rng.uniform(0.5, 1.5, 128).astype(np.float32)).to(device)
    return meta, db


def time_calls(fn, sets, steps, warmup, settle_ms=0.0):
    """Run fn(set) over the rotation; return (wall ms per step, ms per call from HIP events on
    the launch stream around the timed calls; back-to-back calls, so this includes the short
    gaps between them and is never below the kernels' own durations).

    After the `warmup` calls, further untimed calls run until `settle_ms` of wall time has
    passed, so that a workload timed right after another one is measured at its steady clock
    (the first tens of milliseconds of a new load run at a lower shader clock)."""
    import torch

    for i in range(warmup):
        fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    i = 0
    while (time.perf_counter() - t_settle) * 1e3 < settle_ms:
        fn(sets[i % len(sets)])
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    # One event pair around the whole timed region, on the stream the calls are launched on:
    # an event pair around every call would add several microseconds per decode step (each
    # timing event is a packet of its own that waits for the work before it).
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        fn(sets[i % len(sets)])
    end.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    launch_ms = start.elapsed_time(end) / steps
    return wall_ms, launch_ms


def measured_read_ceiling(device, nbytes, sets=4, reps=20):
    """Best rate of a plain streaming read (libpa_probe.so) of `nbytes` bytes, rotating over
    `sets` separate buffers so that no read finds its data in the Infinity Cache; several grid
    sizes, best kept.  Returns (GB/s, description)."""
    import torch

    from deterministic_paged_kv_amd import probe

    n = (nbytes + 15) // 16 * 16
    bufs = [torch.randint(0, 255, (n,), dtype=torch.uint8, device=device) for _ in range(sets)]
    cus = torch.cuda.get_device_properties(device).multi_processor_count
    sink = torch.zeros(16 * cus, dtype=torch.int32, device=device)
    best = (0.0, 0)
    for blocks in (4 * cus, 8 * cus, 16 * cus):
        _, ms = time_calls(lambda buf: probe.read(buf, blocks, sink), bufs, reps, 8, settle_ms=SETTLE_MS)
        best = max(best, (n / (ms * 1e-3) / 1e9, blocks))
    del bufs
    return round(best[0], 1), (f"plain 16-byte-load read of {n} bytes ({sets} buffers rotated, so every read "
                               f"comes from HBM), best of 4/8/16 workgroups per CU ({best[1]} workgroups)")


def measured_mfma_rate(device, reps=10):
    """Rate of independent bf16 MFMAs (libpa_probe.so), 8 wavefronts per CU, for both tile
    shapes; the better is the measured matrix-core ceiling.  Returns (TFLOP/s, description)."""
    import torch

    from deterministic_paged_kv_amd import probe

    cus = torch.cuda.get_device_properties(device).multi_processor_count
    sink = torch.zeros(2 * cus, dtype=torch.float32, device=device)
    rates = {}
    for shape in (16, 32):
        flops = []
        _, ms = time_calls(lambda _: flops.append(probe.mfma(2 * cus, 4096, shape, sink)), [None], reps, 2,
                           settle_ms=SETTLE_MS)
        rates[shape] = flops[-1] / (ms * 1e-3) / 1e12
    best = max(rates, key=rates.get)
    return round(rates[best], 1), (f"independent bf16 MFMAs, 8 wavefronts per CU: 16x16x32 "
                                   f"{rates[16]:.0f} TFLOP/s, 32x32x16 {rates[32]:.0f} TFLOP/s")


def backward_flops(batch, seq, num_q_heads) -> int:
    """Five products over the causally visible pairs of every query head (S = QK^T recomputed,
    dP = dO V^T, dV += P^T dO, dQ = dS K, dK += dS^T Q): 10 * D * Hq * pairs."""
    return 10 * 128 * num_q_heads * batch * (seq * (seq + 1) // 2)


def bench_backward(device, steps, warmup, batch=4, seq=2048, hq=32, hkv=8):
    """Full-prefill backward (training layout): B rows of S tokens at positions 0..S-1, Q/K
    RMSNorm + RoPE, GQA 32/8, bf16 N(0,1) inputs drawn on the device.  The forward's out and lse
    come from one pa_prefill call over the same tokens laid out in pages."""
    import torch

    import deterministic_paged_kv_amd as pa

    gen = torch.Generator(device=device)
    gen.manual_seed(9100)
    rnd = lambda *shape: torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    q, k, v, dout = rnd(batch, hq, seq, 128), rnd(batch, hkv, seq, 128), rnd(batch, hkv, seq, 128), rnd(batch, hq, seq, 128)
    wq = torch.rand(128, generator=gen, device=device) + 0.5
    wk = torch.rand(128, generator=gen, device=device) + 0.5
    npg = seq // 16
    pages = lambda x: x.permute(0, 2, 1, 3).reshape(batch * npg, 16, hkv, 128).contiguous()
    i32 = lambda x: x.to(device=device, dtype=torch.int32)
    indptr = i32(torch.arange(batch + 1) * npg)
    indices = i32(torch.arange(batch * npg))
    last = i32(torch.full((batch,), 16))
    pos = i32(torch.arange(seq).repeat(batch, 1)).contiguous()
    plan = pa.Plan(hq, hkv, max_batch=batch, max_q_len=seq, max_pages_per_row=npg, rms_eps=1e-6)
    kpos = i32(torch.arange(npg * 16).repeat(batch))  # key j of row b at b * npg * 16 + j
    out, lse = pa.prefill(plan, q, pages(k), pages(v), indptr, indices, last, pos, pos, kpos, wq, wk)
    ws = torch.empty(pa.prefill_backward_workspace_size(plan, batch, seq), dtype=torch.uint8, device=device)
    grads = (torch.empty(q.shape, dtype=torch.float32, device=device),
             torch.empty(k.shape, dtype=torch.float32, device=device),
             torch.empty(k.shape, dtype=torch.float32, device=device),
             torch.empty(128, dtype=torch.float32, device=device), torch.empty(128, dtype=torch.float32, device=device))

    def bstep(_):
        pa.prefill_backward(plan, pos, q, k, v, out, lse, dout, q_norm_weight=wq, k_norm_weight=wk, workspace=ws,
                            grads=grads)

    b_wall, b_launch = time_calls(bstep, [None], steps, warmup, settle_ms=SETTLE_MS)
    flops = backward_flops(batch, seq, hq)
    return {"workload": "full_prefill_backward", "batch": batch, "seq_len": seq, "num_q_heads": hq,
            "num_kv_heads": hkv, "steps": steps, "ms_per_call": round(b_wall, 5),
            "value": round(flops / (b_wall * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": round(flops / (b_launch * 1e-3) / 1e12, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(flops / (b_launch * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": None,
                         "kernel": "bwd_prep_kernel + bwd_dq_kernel + bwd_dkdv_kernel + bwd_sum_rows_kernel (whole call)",
                         "algorithmic_flops_per_call": flops, "avg_call_ms": round(b_launch, 5)}}


def affinity_cores() -> int:
    """Cores this process may run on (sched_getaffinity), uncapped."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def host_cores() -> int:
    """Threads the CPU oracle uses: the cores this process may run on, at most 16 (one GPU's
    share of the host's CPUs)."""
    return max(1, min(16, affinity_cores()))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_info(cores) -> dict:
    return {"cores_available": affinity_cores(), "cpu_count": os.cpu_count(), "cpu_model": cpu_model(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"), "threads_used": cores}


def _time_oracle(b, min_seconds, max_reps, threads=None, rows=None):
    """Median wall time of oracle.paged_attention on batch b (or its `rows`), repeated until
    min_seconds of CPU work have been spent (at least 3 runs, at most max_reps), with `threads`
    BLAS threads (default: host_cores())."""
    from threadpoolctl import threadpool_limits

    import oracle

    cores = threads or host_cores()
    args, kwargs = b.oracle_args()
    times = []
    with threadpool_limits(limits=cores):
        while len(times) < 3 or (sum(times) < min_seconds and len(times) < max_reps):
            t0 = time.perf_counter()
            oracle.paged_attention(*args, rows=rows, **kwargs)
            times.append(time.perf_counter() - t0)
    return sorted(times)[len(times) // 2], len(times), sum(times), cores


def cpu_baseline_decode(base, alg_bytes):
    """The CPU oracle (float64 numpy) on the whole decode batch, ~10 s of repeated runs, plus a
    single-thread run on four rows (scaled by those rows' own bytes)."""
    dt, reps, total, cores = _time_oracle(base, 10.0, 40)
    rows = [0, 1, 2, 3]
    sub = 4 * int(sum(base.lengths[r] for r in rows)) * base.num_kv_heads * 128 + \
        4 * len(rows) * base.num_q_heads * 128 + 4 * len(rows) * base.num_q_heads
    dt1, reps1, _, _ = _time_oracle(base, 3.0, 10, threads=1, rows=rows)
    return {"value": round(alg_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"the whole B=32 decode batch (all rows and heads): median of {reps} runs "
                      f"({dt:.2f} s each, {total:.1f} s in all), float64 numpy with {cores} BLAS threads",
            "single_thread": {"value": round(sub / dt1 / 1e9, 4), "unit": "GB/s",
                              "sample": f"rows 0-3 of the same batch, median of {reps1} runs ({dt1:.2f} s each), "
                                        f"one BLAS thread"},
            **host_info(cores)}


def cpu_baseline_prefill(b, flops):
    """The CPU oracle on the whole chunked-prefill batch, ~10 s of repeated runs."""
    dt, reps, total, cores = _time_oracle(b, 10.0, 20)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"the whole chunked-prefill batch: median of {reps} runs ({dt:.2f} s each, "
                      f"{total:.1f} s in all), float64 numpy with {cores} BLAS threads", **host_info(cores)}


def profile_copy():
    """A plain device copy of 1 GiB, for scaling FETCH_SIZE / WRITE_SIZE to bytes."""
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n}))


def _counter_mean(path, counter, kernel_substr):
    """Mean per-dispatch value of one counter over the dispatches whose kernel name contains
    kernel_substr, from a rocprofv3 counter_collection.csv."""
    import csv

    per_dispatch = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]:
            # a counter may come as several rows per dispatch (one per hardware instance)
            per_dispatch[r["Dispatch_Id"]] = per_dispatch.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per_dispatch:
        raise SystemExit(f"no {counter} rows for {kernel_substr!r} in {path}")
    return sum(per_dispatch.values()) / len(per_dispatch), len(per_dispatch)


def ingest_counters(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """HBM bytes per decode launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by
    what the same counter reads for a plain 1 GiB copy (which moves exactly 1 GiB each way)."""
    import workloads

    copy_bytes = 1 << 30
    cf, _ = _counter_mean(copy_fetch_csv, "FETCH_SIZE", "copyBuffer")
    cw, _ = _counter_mean(copy_write_csv, "WRITE_SIZE", "copyBuffer")
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    # one decode call = the stream kernel + the combining kernel
    fk, nf = _counter_mean(fetch_csv, "FETCH_SIZE", "decode_stream_kernel")
    wk, nw = _counter_mean(write_csv, "WRITE_SIZE", "decode_stream_kernel")
    fk2, _ = _counter_mean(fetch_csv, "FETCH_SIZE", "decode_combine_kernel")
    wk2, _ = _counter_mean(write_csv, "WRITE_SIZE", "decode_combine_kernel")
    fk, wk = fk + fk2, wk + wk2
    fetch = fk * 1024.0 * f_scale
    write = wk * 1024.0 * w_scale
    alg = decode_bytes(workloads.qwen3_8b_decode(canary=False))
    doc = {
        "kernel": "decode_stream_kernel + decode_combine_kernel", "workload": "qwen3_8b_decode",
        "source_hash": source_hash(DECODE_SOURCES),
        "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
        "dispatches": [nf, nw],
        "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1),
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        "hbm_bytes_per_launch": int(round(fetch + write)),
        "algorithmic_bytes_per_launch": alg,
        "traffic_over_algorithmic": round((fetch + write) / alg, 4),
    }
    out = os.path.join(ROOT, "profiles", "decode_qwen3_8b_counters.json")
    with open(out, "w") as fh:
        json.dump(doc, fh, indent=1)
        fh.write("\n")
    print(json.dumps(doc))


# SQ counters of the attention kernel, two passes (at most 8 SQ counters per pass)
PREFILL_SQ_PASSES = [
    ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
     "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS"],
    ["SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES",
     "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_WAIT_INST_LDS"],
]


def ingest_prefill_counters(sq1_csv, sq2_csv, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """Per-call counters of the chunked-prefill kernels (the bench.py prefill workload): SQ
    counters of attend_kernel (mean per dispatch) and HBM bytes of both kernels from FETCH_SIZE /
    WRITE_SIZE scaled by a plain 1 GiB copy.  Writes profiles/prefill_chunked_counters.json."""
    import workloads

    copy_bytes = 1 << 30
    cf, _ = _counter_mean(copy_fetch_csv, "FETCH_SIZE", "copyBuffer")
    cw, _ = _counter_mean(copy_write_csv, "WRITE_SIZE", "copyBuffer")
    f_scale, w_scale = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)
    sq = {}
    for path, names in ((sq1_csv, PREFILL_SQ_PASSES[0]), (sq2_csv, PREFILL_SQ_PASSES[1])):
        for c in names:
            sq[c], _ = _counter_mean(path, c, "attend_kernel")
    hbm = {}
    for k in ("attend_kernel", "prologue_kernel"):
        fk, _ = _counter_mean(fetch_csv, "FETCH_SIZE", k)
        wk, _ = _counter_mean(write_csv, "WRITE_SIZE", k)
        hbm[k] = {"fetch_bytes": int(fk * 1024.0 * f_scale), "write_bytes": int(wk * 1024.0 * w_scale)}
    pb = workloads.chunked_prefill(canary=False)
    flops = prefill_flops(pb)
    mfma_flops = sq["SQ_INSTS_MFMA"] * 32768  # every MFMA of the kernel is v_mfma_f32_32x32x16_bf16
    doc = {
        "kernels": PREFILL_KERNELS, "workload": "chunked_prefill", "source_hash": source_hash(PREFILL_SOURCES),
        "attend_sq_per_dispatch": {k: int(round(v)) for k, v in sq.items()},
        "attend_derived": {
            # SQ_WAVE_CYCLES and the SQ_ACTIVE/WAIT counters count in units of 4 cycles
            "mfma_busy_cycles_per_mfma": round(sq["SQ_VALU_MFMA_BUSY_CYCLES"] / sq["SQ_INSTS_MFMA"], 2),
            "mfma_flops_over_algorithmic": round(mfma_flops / flops, 4),
            "valu_insts_per_mfma": round(sq["SQ_INSTS_VALU"] / sq["SQ_INSTS_MFMA"], 2),
            "lds_insts_per_mfma": round(sq["SQ_INSTS_LDS"] / sq["SQ_INSTS_MFMA"], 2),
            "salu_insts_per_mfma": round(sq["SQ_INSTS_SALU"] / sq["SQ_INSTS_MFMA"], 2),
            "lds_bank_conflict_over_active": round(sq["SQ_LDS_BANK_CONFLICT"] / max(sq["SQ_LDS_IDX_ACTIVE"], 1), 4),
            "wave_time_waiting_frac": round(sq["SQ_WAIT_ANY"] / sq["SQ_WAVE_CYCLES"], 4),
            "wave_time_issue_stalled_frac": round(sq["SQ_WAIT_INST_ANY"] / sq["SQ_WAVE_CYCLES"], 4),
            "wave_time_issuing_frac": round(sq["SQ_ACTIVE_INST_ANY"] / sq["SQ_WAVE_CYCLES"], 4),
        },
        "hbm_bytes_per_call": hbm,
        "hbm_bytes_per_call_total": sum(v["fetch_bytes"] + v["write_bytes"] for v in hbm.values()),
        "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1),
        "algorithmic_flops_per_call": flops,
    }
    with open(PREFILL_COUNTERS, "w") as fh:
        json.dump(doc, fh, indent=1)
        fh.write("\n")
    print(json.dumps(doc))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--profile-copy", action="store_true")
    ap.add_argument("--decode-only", action="store_true", help="skip prefill and the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true", help="time only the chunked prefill")
    ap.add_argument("--backward-only", action="store_true", help="time only the full-prefill backward")
    ap.add_argument("--ingest-counters", nargs=4, metavar="CSV")
    ap.add_argument("--ingest-prefill-counters", nargs=6, metavar="CSV")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters)
        return
    if args.ingest_prefill_counters:
        ingest_prefill_counters(*args.ingest_prefill_counters)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              f"multi-GPU path: rows and heads shard across GPUs with no exchange, see the design notes.",
              file=sys.stderr)
        sys.exit(2)
    if args.profile_copy:
        profile_copy()
        return

    import numpy as np
    import torch

    import deterministic_paged_kv_amd as pa
    import workloads
    from tests._paged import DeviceBatch

    device = "cuda:0"
    torch.cuda.set_device(0)
    if args.backward_only:
        print(json.dumps({"prefill_backward": bench_backward(device, max(10, args.steps // 10), 3)}), flush=True)
        return
    print("[bench] building inputs", file=sys.stderr, flush=True)
    base = workloads.qwen3_8b_decode(canary=False)
    sets = [device_rotation(base, i, device) for i in range(ROTATIONS)]
    plan = pa.Plan(16, 4, max_batch=32, max_q_len=1, max_pages_per_row=256, rms_eps=base.eps)
    out = torch.empty_like(sets[0].q)
    lse = torch.empty(out.shape[:3], dtype=torch.float32, device=device)
    rep = pa.validate_metadata(plan, batch=32, q_len=1, num_pages=base.num_pages,
                               kv_indptr=sets[0].kv_indptr, kv_indices=sets[0].kv_indices,
                               kv_last_page_len=sets[0].kv_last_page_len, cache_position=sets[0].cache_position,
                               query_position_ids=sets[0].query_position_ids,
                               key_position_ids=sets[0].key_position_ids)
    if rep["code"] != 0:
        raise RuntimeError(f"metadata rejected: {rep}")

    def step(db):
        pa.decode(plan, *db.args(), out=out, lse=lse)

    ws = pa.decode_workspace(plan, 32, device=device)

    def step_multi(db):
        pa.decode(plan, *db.args(), out=out, lse=lse, workspace=ws)

    print("[bench] timing decode", file=sys.stderr, flush=True)
    dsteps = 2 if args.prefill_only else args.steps
    # the W warmup steps, then untimed steps until SETTLE_MS have passed (the first tens of
    # milliseconds of a new load run at a lower shader clock), then exactly K timed steps
    wall_ms, launch_ms = time_calls(step_multi, sets, dsteps, 0 if args.prefill_only else args.warmup,
                                    settle_ms=0.0 if args.prefill_only else SETTLE_MS)
    unit_wall_ms, unit_launch_ms = time_calls(step, sets, dsteps, 0 if args.prefill_only else args.warmup,
                                              settle_ms=0.0 if args.prefill_only else SETTLE_MS)
    alg = decode_bytes(base)
    value = alg / (wall_ms * 1e-3) / 1e9
    achieved = alg / (launch_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3_8b_decode", "batch": 32, "q_len": 1, "num_q_heads": 16, "num_kv_heads": 4,
                   "head_dim": 128, "page_size": 16, "kv_len": "U{512..4096}", "total_keys": int(np.sum(base.lengths)),
                   "pool_pages": base.num_pages, "kv_pool_rotation": ROTATIONS, "split_kv": "disabled"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_from_profile(alg),
                     "kernel": "decode_stream_kernel + decode_combine_kernel (one call)",
                     "algorithmic_bytes_per_launch": alg, "avg_launch_ms": round(launch_ms, 5)},
        # the same reduction tree in one workgroup per (row, KV head), no workspace:
        # bit-identical results (tested)
        "decode_one_workgroup_per_unit": {
            "value": round(alg / (unit_wall_ms * 1e-3) / 1e9, 2), "unit": "GB/s",
            "ms_per_step": round(unit_wall_ms, 5), "kernel": "decode_unit_kernel",
            "avg_launch_ms": round(unit_launch_ms, 5),
            "frac": round(alg / (unit_launch_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }

    if not args.prefill_only:
        # the measured read ceiling at this call's size, beside the published peak
        print("[bench] measuring the read ceiling", file=sys.stderr, flush=True)
        ceil_gbs, ceil_how = measured_read_ceiling(device, alg)
        result["roofline"].update({"peak_measured": ceil_gbs, "frac_measured": round(achieved / ceil_gbs, 4),
                                   "peak_measured_how": ceil_how})

    if not args.decode_only and not args.prefill_only:
        # Long-context low-batch decode (B=1, L=131,072): the 16-stream tree against the
        # fixed-chunk policy, which cuts the row into 1,024-token chunks (128 chunks).
        print("[bench] timing long-context decode", file=sys.stderr, flush=True)
        lmeta, ldb = long_context_set(1, 131072, device)
        lout = torch.empty_like(ldb.q)
        llse = torch.empty(lout.shape[:3], dtype=torch.float32, device=device)
        lalg = decode_bytes(lmeta)
        long_result = {"workload": "long_context_decode", "batch": 1, "kv_len": 131072, "num_q_heads": 32,
                       "num_kv_heads": 8, "algorithmic_bytes_per_call": lalg}
        for name, policy, chunk in (("split_disabled", pa.PA_SPLIT_DISABLED, 0),
                                    ("split_fixed_1024", pa.PA_SPLIT_FIXED, 1024)):
            lplan = pa.Plan(32, 8, max_batch=1, max_q_len=1, max_pages_per_row=8192, rms_eps=1e-6,
                            split_policy=policy, split_chunk_tokens=chunk)
            lws = pa.decode_workspace(lplan, 1, device=device)

            def lstep(db, lplan=lplan, lws=lws):
                pa.decode(lplan, *db.args(), out=lout, lse=llse, workspace=lws)

            l_wall, l_launch = time_calls(lstep, [ldb], 20, 3, settle_ms=SETTLE_MS)
            long_result[name] = {"ms_per_call": round(l_launch, 5),
                                 "value": round(lalg / (l_launch * 1e-3) / 1e9, 2), "unit": "GB/s",
                                 "frac": round(lalg / (l_launch * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        result["long_context_decode"] = long_result
        del ldb
        # The whole long-context grid: B in {1, 2, 4} x L in {32,768, 65,536, 131,072}, one pool.
        print("[bench] timing the long-context grid", file=sys.stderr, flush=True)
        pool = long_context_pool(device)
        sweep = []
        for lb in (1, 2, 4):
            for ll in (32768, 65536, 131072):
                smeta, sdb = long_context_set(lb, ll, device, pool=pool)
                sout = torch.empty_like(sdb.q)
                slse = torch.empty(sout.shape[:3], dtype=torch.float32, device=device)
                salg = decode_bytes(smeta)
                entry = {"batch": lb, "kv_len": ll, "algorithmic_bytes_per_call": salg}
                for name, policy, chunk in (("split_disabled", pa.PA_SPLIT_DISABLED, 0),
                                            ("split_fixed_1024", pa.PA_SPLIT_FIXED, 1024)):
                    splan = pa.Plan(32, 8, max_batch=lb, max_q_len=1, max_pages_per_row=ll // 16, rms_eps=1e-6,
                                    split_policy=policy, split_chunk_tokens=chunk)
                    sws = pa.decode_workspace(splan, lb, device=device)

                    def sstep(db, splan=splan, sws=sws):
                        pa.decode(splan, *db.args(), out=sout, lse=slse, workspace=sws)

                    _, s_launch = time_calls(sstep, [sdb], 20, 3, settle_ms=SETTLE_MS)
                    entry[name] = {"ms_per_call": round(s_launch, 5),
                                   "value": round(salg / (s_launch * 1e-3) / 1e9, 2), "unit": "GB/s",
                                   "frac": round(salg / (s_launch * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
                    splan.close()
                sweep.append(entry)
                del sdb
        result["long_context_grid"] = sweep
        del pool

    if not args.decode_only:
        print("[bench] timing prefill", file=sys.stderr, flush=True)
        pb = workloads.chunked_prefill(canary=False)
        pdb = DeviceBatch(pb, device)
        pplan = pa.Plan(32, 8, max_batch=4, max_q_len=512, max_pages_per_row=256, rms_eps=pb.eps)
        pout = torch.empty_like(pdb.q)
        plse = torch.empty(pout.shape[:3], dtype=torch.float32, device=device)
        ws = torch.empty(pa.prefill_workspace_size(pplan, 4, 512, pb.nnz), dtype=torch.uint8, device=device)

        def pstep(db):
            pa.prefill(pplan, *db.args(), out=pout, lse=plse, workspace=ws)

        psteps = max(20, args.steps // 4)
        # Cold: the calls cycle over PREFILL_ROTATIONS sets (same lengths and positions, other
        # pages and contents; about 420 MB of q, K and V in all), so no call finds its inputs in
        # the 256 MB Infinity Cache.  Warm: one set, called again and again.
        psets = [device_rotation(pb, i, device) for i in range(PREFILL_ROTATIONS)]
        p_wall, p_launch = time_calls(pstep, psets, psteps, args.warmup, settle_ms=SETTLE_MS)
        _, p_warm = time_calls(pstep, [pdb], psteps, args.warmup, settle_ms=SETTLE_MS)
        del psets
        flops = prefill_flops(pb)
        print("[bench] measuring the matrix-core rate", file=sys.stderr, flush=True)
        mfma_rate, mfma_how = measured_mfma_rate(device)
        p_ach = flops / (p_launch * 1e-3) / 1e12
        result["prefill"] = {
            "workload": "chunked_prefill", "batch": 4, "q_len": 512, "prefixes": [0, 1024, 2048, 3584],
            "num_q_heads": 32, "num_kv_heads": 8, "steps": psteps, "input_rotation": PREFILL_ROTATIONS,
            "warm_avg_call_ms": round(p_warm, 5), "ms_per_call": round(p_wall, 5),
            "value": round(flops / (p_wall * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": round(p_ach, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(p_ach / MFMA_BF16_PEAK_TFLOPS, 4),
                         "peak_measured": mfma_rate, "frac_measured": round(p_ach / mfma_rate, 4),
                         "peak_measured_how": mfma_how,
                         "traffic": None, "kernel": PREFILL_KERNELS + " (whole call)",
                         "algorithmic_flops_per_call": flops, "avg_call_ms": round(p_launch, 5)},
        }
        pc = prefill_counters_from_profile()
        if pc is not None:
            # HBM bytes of both kernels per call (counters of the same source), and the attention
            # kernel's instruction mix: where the time goes, against the MFMA-bound target
            result["prefill"]["roofline"]["traffic"] = pc["hbm_bytes_per_call_total"]
            result["prefill"]["counters"] = {"source": os.path.relpath(PREFILL_COUNTERS, ROOT),
                                             **pc["attend_derived"]}
        if not args.prefill_only:
            print("[bench] timing the full-prefill backward", file=sys.stderr, flush=True)
            result["prefill_backward"] = bench_backward(device, max(10, args.steps // 10), 3)
        if not args.no_cpu_baseline:
            print("[bench] timing the CPU oracle (decode, then prefill)", file=sys.stderr, flush=True)
            result["cpu_baseline"] = cpu_baseline_decode(base, alg)
            result["prefill"]["cpu_baseline"] = cpu_baseline_prefill(pb, flops)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
