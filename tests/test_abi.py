"""The C-ABI library loads, exports every symbol include/pa.h declares, and rejects bad host
arguments before touching the GPU.  CPU only: nothing here launches a kernel."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from deterministic_paged_kv_amd import binding

    return binding.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("pa_plan", "pa_plan_destroy", "pa_validate_metadata", "pa_decode", "pa_prefill",
                     "pa_decode_workspace_size", "pa_prefill_workspace_size", "pa_status_string"):
        assert required in names


def test_every_declared_symbol_is_exported_and_bound(lib):
    from deterministic_paged_kv_amd import binding

    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in binding.SIGNATURES, name


def test_binding_argument_counts_match_the_header():
    """Every binding signature takes as many arguments as the header's declaration lists."""
    from deterministic_paged_kv_amd import binding

    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for name, params in re.findall(r"\b(pa_[a-z_]+)\s*\(([^;{]*?)\)\s*;", text):
        if name not in binding.SIGNATURES:
            continue
        n = 0 if params.strip() in ("", "void") else params.count(",") + 1
        assert len(binding.SIGNATURES[name][1]) == n, (name, n, len(binding.SIGNATURES[name][1]))


def test_status_strings(lib):
    from deterministic_paged_kv_amd import binding

    for code, name in binding.STATUS.items():
        assert lib.pa_status_string(code).decode() == name
    assert lib.pa_status_string(12345).decode() == "PA_ERR_UNKNOWN"


def _plan(lib, hq=16, hkv=4, d=128, ps=16, mb=1, mq=1, mp=1, theta=1e6, scale=1.0, eps=1e-6, split=0, chunk=0):
    h = ctypes.c_void_p()
    st = lib.pa_plan(hq, hkv, d, ps, mb, mq, mp, theta, scale, eps, split, chunk, ctypes.byref(h))
    assert h.value is None  # written only on success; none of these cases succeed
    return st


def test_plan_fails_closed_on_host_arguments(lib):
    assert _plan(lib, d=64) == -2
    assert _plan(lib, ps=32) == -2
    assert _plan(lib, theta=1e4) == -2
    assert _plan(lib, scale=2.0) == -2
    assert _plan(lib, split=1) == -2          # fixed split without a chunk size
    assert _plan(lib, split=1, chunk=8) == -2     # chunk below one page
    assert _plan(lib, split=1, chunk=40) == -2    # chunk not a multiple of the page size
    assert _plan(lib, split=1, chunk=-16) == -2
    assert _plan(lib, split=2) == -2          # auto split: rejected
    assert _plan(lib, split=2, chunk=64) == -2
    assert _plan(lib, split=3) == -2          # unknown policy
    assert _plan(lib, hq=16, hkv=3) == -4     # head ratio
    assert _plan(lib, hq=34, hkv=2) == -4     # group of 17 > 16
    assert _plan(lib, hq=0) == -1
    assert _plan(lib, mb=0) == -1
    assert _plan(lib, eps=0.0) == -1
    assert _plan(lib, mp=1 << 21) == -3       # positions past 2^24
    assert _plan(lib, mb=1 << 23) == -3       # (row, KV head) units past 2^24
    assert _plan(lib, split=1, chunk=16, mp=4097) == -3   # 4,097 chunks of one page per row
    assert _plan(lib, split=1, chunk=32, mp=8193) == -3   # 4,097 chunks of two pages
    assert lib.pa_plan(16, 4, 128, 16, 1, 1, 1, 1e6, 1.0, 1e-6, 0, 0, None) == -1


def test_calls_without_a_plan_fail_closed(lib):
    null = None
    assert lib.pa_decode(null, 1, 1, 1, 0, *([null] * 14), 0, null) == -1
    assert lib.pa_decode_workspace_size(null, 1, ctypes.byref(ctypes.c_size_t())) == -1
    assert lib.pa_prefill(null, 1, 1, 1, 0, *([null] * 14), 0, null) == -1
    from deterministic_paged_kv_amd import binding

    rep = binding.ValidationReport()
    assert lib.pa_validate_metadata(null, 1, 1, 1, 0, *([null] * 7), ctypes.byref(rep)) == -1
    assert rep.code == -1
    n = ctypes.c_size_t()
    assert lib.pa_prefill_workspace_size(null, 1, 1, 0, ctypes.byref(n)) == -1
    assert lib.pa_plan_destroy(null) == 0


def test_product_path_does_not_import_the_oracle():
    import subprocess
    import sys

    code = ("import sys, deterministic_paged_kv_amd as d; d.load(); "
            "assert not any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules), 'oracle imported'")
    subprocess.run([sys.executable, "-c", code], check=True, cwd=ROOT)
    for dirpath, _, files in os.walk(os.path.join(ROOT, "deterministic_paged_kv_amd")):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), f


def test_csr_builder_rejects_bad_sizes_before_any_launch(lib):
    """pa_build_csr checks its host scalars and pointers before it launches anything."""
    p = ctypes.c_void_p(16)  # never dereferenced: every call below fails its host checks
    assert lib.pa_build_csr(-1, 4, p, p, p, p, p, None) == -1     # negative batch
    assert lib.pa_build_csr(2, 0, p, p, p, p, p, None) == -1      # width 0
    assert lib.pa_build_csr(2, 1 << 28, p, p, p, p, p, None) == -1  # width * 16 overflows int32
    assert lib.pa_build_csr(1 << 16, 1 << 16, p, p, p, p, p, None) == -1  # B * width overflows int32
    assert lib.pa_build_csr(2, 4, p, p, None, p, p, None) == -1   # no indptr
    assert lib.pa_build_csr(2, 4, None, p, p, p, p, None) == -1   # no table for B > 0
    assert lib.pa_build_csr(2, 4, p, None, p, p, p, None) == -1   # no lengths
    assert lib.pa_build_csr(2, 4, p, p, p, None, p, None) == -1   # no indices
    assert lib.pa_build_csr(2, 4, p, p, p, p, None, None) == -1   # no last_page_len


def test_width_bucket_is_the_next_power_of_two(lib):
    """Plans keyed by a power-of-two width ("flashinfer_fa2 backend for NVIDIA Ada (SM89)",
    "Design notes"): the smallest power of two not below the width."""
    out = ctypes.c_int32()
    for w, want in [(1, 1), (2, 2), (3, 4), (16, 16), (17, 32), (40, 64), (4096, 4096), (4097, 8192),
                    (1 << 30, 1 << 30)]:
        assert lib.pa_width_bucket(w, ctypes.byref(out)) == 0
        assert out.value == want, (w, out.value)
    assert lib.pa_width_bucket(0, ctypes.byref(out)) == -1
    assert lib.pa_width_bucket((1 << 30) + 1, ctypes.byref(out)) == -1
    assert lib.pa_width_bucket(8, None) == -1


def test_backward_without_a_plan_fails_closed(lib):
    """pa_prefill_backward and its workspace query check the plan before anything else."""
    p = ctypes.c_void_p(16)  # never dereferenced: both calls fail the plan check
    assert lib.pa_prefill_backward(None, 1, 1, p, p, p, p, None, None, p, p, p, p, p, p, None, None,
                                   p, 1 << 20, None) == -1
    n = ctypes.c_size_t()
    assert lib.pa_prefill_backward_workspace_size(None, 1, 1, ctypes.byref(n)) == -1


def test_probe_library_exports_its_header():
    """libpa_probe.so (the measurement kernels of include/pa_probe.h) exports every declared
    symbol with the binding's argument count, and rejects bad host arguments before any launch."""
    from deterministic_paged_kv_amd import probe

    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "pa_probe.h")).read(), flags=re.S)
    decls = re.findall(r"\b(pa_[a-z_]+)\s*\(([^;{]*?)\)\s*;", text)
    assert {n for n, _ in decls} == set(probe.SIGNATURES)
    plib = probe.load()
    for name, params in decls:
        assert hasattr(plib, name)
        assert len(probe.SIGNATURES[name][1]) == params.count(",") + 1, name
    p = ctypes.c_void_p(16)  # never dereferenced: every call below fails its host checks
    assert plib.pa_probe_read(p, 0, 1, p, None) == -1          # no bytes
    assert plib.pa_probe_read(p, 24, 1, p, None) == -1         # not a multiple of 16
    assert plib.pa_probe_read(p, 32, 0, p, None) == -1         # no workgroups
    assert plib.pa_probe_read(None, 32, 1, p, None) == -1
    assert plib.pa_probe_mfma(1, 1, 8, p, None) == -1          # unknown shape
    assert plib.pa_probe_mfma(0, 1, 16, p, None) == -1
    assert plib.pa_probe_mfma(1, 0, 16, p, None) == -1
    assert plib.pa_probe_mfma(1, 1, 16, None, None) == -1
