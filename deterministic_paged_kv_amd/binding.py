"""Thin ctypes binding over libpa.so (include/pa.h).

Argument marshalling only: torch tensors become device pointers, shapes become the
host scalars the C ABI takes, and the current torch stream is passed as the HIP
stream.  Every step of the attention runs in the library's HIP kernels; there is
no fallback of any kind, and a missing or incomplete library raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpa.so")

PA_SPLIT_DISABLED = 0
PA_SPLIT_FIXED = 1
HEAD_DIM = 128
PAGE_SIZE = 16

# name -> (restype, argtypes), in the order of include/pa.h
_i32, _f32, _p, _sz = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class ValidationReport(ctypes.Structure):
    _fields_ = [("code", ctypes.c_int32), ("row", ctypes.c_int32), ("index", ctypes.c_int64),
                ("value", ctypes.c_int64)]


SIGNATURES = {
    "pa_status_string": (ctypes.c_char_p, [_i32]),
    "pa_plan": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _f32, _f32, _i32, _i32, ctypes.POINTER(_p)]),
    "pa_plan_destroy": (_i32, [_p]),
    "pa_validate_metadata": (_i32, [_p, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p,
                                    ctypes.POINTER(ValidationReport)]),
    "pa_decode": (_i32, [_p, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz,
                         _p]),
    "pa_decode_no_alloc": (_i32, [_p, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                  _p]),
    "pa_decode_workspace_size": (_i32, [_p, _i32, ctypes.POINTER(_sz)]),
    "pa_prefill_workspace_size": (_i32, [_p, _i32, _i32, _i32, ctypes.POINTER(_sz)]),
    "pa_prefill": (_i32, [_p, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz,
                          _p]),
    "pa_build_csr": (_i32, [_i32, _i32, _p, _p, _p, _p, _p, _p]),
    "pa_prefill_backward_workspace_size": (_i32, [_p, _i32, _i32, ctypes.POINTER(_sz)]),
    "pa_prefill_backward": (_i32, [_p, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                   _sz, _p]),
    "pa_width_bucket": (_i32, [_i32, ctypes.POINTER(_i32)]),
}

STATUS = {
    0: "PA_OK", -1: "PA_ERR_INVALID_ARGUMENT", -2: "PA_ERR_UNSUPPORTED", -3: "PA_ERR_CAPACITY",
    -4: "PA_ERR_HEAD_RATIO", -5: "PA_ERR_INDPTR", -6: "PA_ERR_PAGE_OOB", -7: "PA_ERR_DUPLICATE_PAGE",
    -8: "PA_ERR_LAST_PAGE_LEN", -9: "PA_ERR_KEY_POSITION", -10: "PA_ERR_QUERY_POSITION",
    -11: "PA_ERR_CACHE_POSITION", -12: "PA_ERR_WORKSPACE", -13: "PA_ERR_HIP",
}

_lib = None


class PagedAttentionError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = int(status)
        self.name = STATUS.get(self.status, f"status {status}")
        super().__init__(f"{where}: {self.name}")


def load():
    """Load libpa.so and bind every entry point of include/pa.h; raises if any is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)  # AttributeError if the symbol is absent
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != 0:
        raise PagedAttentionError(status, where)


def status_string(status: int) -> str:
    return load().pa_status_string(int(status)).decode()


# ----------------------------------------------------------------------------------------
# tensor marshalling helpers
# ----------------------------------------------------------------------------------------

def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t, name, dtype, ndim=None, shape=None):
    import torch

    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    del torch
    return t


def _stream(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class Plan:
    """An immutable plan: head counts, capacities and the RoPE cos/sin table on the device."""

    def __init__(self, num_q_heads: int, num_kv_heads: int, *, max_batch: int, max_q_len: int,
                 max_pages_per_row: int, head_dim: int = HEAD_DIM, page_size: int = PAGE_SIZE,
                 rope_theta: float = 1e6, rope_scale: float = 1.0, rms_eps: float = 1e-6,
                 split_policy: int = PA_SPLIT_DISABLED, split_chunk_tokens: int = 0):
        lib = load()
        h = ctypes.c_void_p()
        _check(lib.pa_plan(num_q_heads, num_kv_heads, head_dim, page_size, max_batch, max_q_len,
                           max_pages_per_row, rope_theta, rope_scale, rms_eps, split_policy,
                           split_chunk_tokens, ctypes.byref(h)), "pa_plan")
        self.handle = h
        self.num_q_heads = num_q_heads
        self.num_kv_heads = num_kv_heads
        self.max_batch = max_batch
        self.max_q_len = max_q_len
        self.max_pages_per_row = max_pages_per_row
        self.split_policy = split_policy
        self.split_chunk_tokens = split_chunk_tokens if split_policy == PA_SPLIT_FIXED else 0

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            _check(load().pa_plan_destroy(self.handle), "pa_plan_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _metadata(plan, q, k_cache, v_cache, kv_indptr, kv_indices, kv_last_page_len, cache_position,
              query_position_ids, key_position_ids):
    import torch

    _need(q, "q", torch.bfloat16, 4)
    B, Hq, Sq, D = q.shape
    if Hq != plan.num_q_heads or D != HEAD_DIM:
        raise ValueError(f"q shape {tuple(q.shape)} does not match the plan")
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    if tuple(k_cache.shape[1:]) != (PAGE_SIZE, plan.num_kv_heads, HEAD_DIM):
        raise ValueError(f"k_cache shape {tuple(k_cache.shape)} does not match the plan")
    _need(v_cache, "v_cache", torch.bfloat16, shape=k_cache.shape)
    _need(kv_indptr, "kv_indptr", torch.int32, shape=(B + 1,))
    _need(kv_indices, "kv_indices", torch.int32, 1)
    _need(kv_last_page_len, "kv_last_page_len", torch.int32, shape=(B,))
    _need(cache_position, "cache_position", torch.int32, shape=(B, Sq))
    _need(query_position_ids, "query_position_ids", torch.int32, shape=(B, Sq))
    nnz = int(kv_indices.shape[0])
    _need(key_position_ids, "key_position_ids", torch.int32, shape=(nnz * PAGE_SIZE,))
    return B, Sq, int(k_cache.shape[0]), nnz


def validate_metadata(plan: Plan, *, batch: int, q_len: int, num_pages: int, kv_indptr, kv_indices,
                      kv_last_page_len, cache_position, query_position_ids, key_position_ids,
                      stream=None) -> dict:
    """Run pa_validate_metadata; returns {'code', 'status', 'row', 'index', 'value'} (no raise)."""
    import torch

    _need(kv_indptr, "kv_indptr", torch.int32, shape=(batch + 1,))
    _need(kv_indices, "kv_indices", torch.int32, 1)
    _need(kv_last_page_len, "kv_last_page_len", torch.int32, shape=(batch,))
    _need(cache_position, "cache_position", torch.int32, shape=(batch, q_len))
    _need(query_position_ids, "query_position_ids", torch.int32, shape=(batch, q_len))
    nnz = int(kv_indices.shape[0])
    _need(key_position_ids, "key_position_ids", torch.int32, shape=(nnz * PAGE_SIZE,))
    rep = ValidationReport()
    code = load().pa_validate_metadata(plan.handle, batch, q_len, num_pages, nnz, _ptr(kv_indptr),
                                       _ptr(kv_indices), _ptr(kv_last_page_len), _ptr(cache_position),
                                       _ptr(query_position_ids), _ptr(key_position_ids), _stream(stream),
                                       ctypes.byref(rep))
    return {"code": int(code), "status": STATUS.get(int(code), str(code)), "row": int(rep.row),
            "index": int(rep.index), "value": int(rep.value)}


def decode_workspace_size(plan: Plan, batch: int) -> int:
    n = ctypes.c_size_t()
    _check(load().pa_decode_workspace_size(plan.handle, batch, ctypes.byref(n)), "pa_decode_workspace_size")
    return int(n.value)


def decode_workspace(plan: Plan, batch: int, device="cuda"):
    """A workspace for pa_decode's multi-compute-unit schedule, sized for the plan's split
    policy (needs no initialisation and can be reused by calls that do not overlap in time;
    a PA_SPLIT_FIXED plan requires one)."""
    import torch

    return torch.empty(decode_workspace_size(plan, batch), dtype=torch.uint8, device=device)


def decode(plan: Plan, q, k_cache, v_cache, kv_indptr, kv_indices, kv_last_page_len, cache_position,
           query_position_ids, key_position_ids, q_norm_weight=None, k_norm_weight=None, out=None, lse=None,
           workspace=None, stream=None):
    """pa_decode.  q [B, Hq, 1, 128] bf16; returns (out [B, Hq, 1, 128] bf16, lse [B, Hq, 1] fp32).

    workspace: None for the one-workgroup-per-(row, KV head) schedule, or a uint8 device tensor
    from decode_workspace() (any contents) for the multi-compute-unit schedule (same bits)."""
    import torch

    B, Sq, num_pages, nnz = _metadata(plan, q, k_cache, v_cache, kv_indptr, kv_indices, kv_last_page_len,
                                      cache_position, query_position_ids, key_position_ids)
    if q_norm_weight is not None:
        _need(q_norm_weight, "q_norm_weight", torch.float32, shape=(HEAD_DIM,))
    if k_norm_weight is not None:
        _need(k_norm_weight, "k_norm_weight", torch.float32, shape=(HEAD_DIM,))
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16, shape=q.shape)
    _need(lse, "lse", torch.float32, shape=q.shape[:3])
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1)
        ws_bytes = int(workspace.numel())
    _check(load().pa_decode(plan.handle, B, Sq, num_pages, nnz, _ptr(kv_indptr), _ptr(kv_indices),
                            _ptr(kv_last_page_len), _ptr(cache_position), _ptr(query_position_ids),
                            _ptr(key_position_ids), _ptr(q), _ptr(k_cache),
                            _ptr(v_cache), _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(out), _ptr(lse),
                            _ptr(workspace), ws_bytes, _stream(stream)), "pa_decode")
    return out, lse


def decode_no_alloc(plan: Plan, q, k_cache, v_cache, kv_indptr, kv_indices, kv_last_page_len, cache_position,
                    query_position_ids, key_position_ids, q_norm_weight=None, k_norm_weight=None, *, out, lse,
                    stream=None):
    """pa_decode_no_alloc: the multi-compute-unit decode with the library's own scratch (no
    workspace, no allocation).  out and lse must be given (nothing is allocated here either);
    calls that overlap in time on one device race on the shared scratch."""
    import torch

    B, Sq, num_pages, nnz = _metadata(plan, q, k_cache, v_cache, kv_indptr, kv_indices, kv_last_page_len,
                                      cache_position, query_position_ids, key_position_ids)
    if q_norm_weight is not None:
        _need(q_norm_weight, "q_norm_weight", torch.float32, shape=(HEAD_DIM,))
    if k_norm_weight is not None:
        _need(k_norm_weight, "k_norm_weight", torch.float32, shape=(HEAD_DIM,))
    _need(out, "out", torch.bfloat16, shape=q.shape)
    _need(lse, "lse", torch.float32, shape=q.shape[:3])
    _check(load().pa_decode_no_alloc(plan.handle, B, Sq, num_pages, nnz, _ptr(kv_indptr), _ptr(kv_indices),
                                     _ptr(kv_last_page_len), _ptr(cache_position), _ptr(query_position_ids),
                                     _ptr(key_position_ids), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(out), _ptr(lse),
                                     _stream(stream)), "pa_decode_no_alloc")
    return out, lse


def prefill_workspace_size(plan: Plan, batch: int, q_len: int, num_indices: int) -> int:
    n = ctypes.c_size_t()
    _check(load().pa_prefill_workspace_size(plan.handle, batch, q_len, num_indices, ctypes.byref(n)),
           "pa_prefill_workspace_size")
    return int(n.value)


def prefill(plan: Plan, q, k_cache, v_cache, kv_indptr, kv_indices, kv_last_page_len, cache_position,
            query_position_ids, key_position_ids, q_norm_weight=None, k_norm_weight=None, out=None, lse=None,
            workspace=None, stream=None):
    """pa_prefill.  q [B, Hq, Sq, 128] bf16; returns (out [B, Hq, Sq, 128] bf16, lse [B, Hq, Sq] fp32)."""
    import torch

    B, Sq, num_pages, nnz = _metadata(plan, q, k_cache, v_cache, kv_indptr, kv_indices, kv_last_page_len,
                                      cache_position, query_position_ids, key_position_ids)
    if q_norm_weight is not None:
        _need(q_norm_weight, "q_norm_weight", torch.float32, shape=(HEAD_DIM,))
    if k_norm_weight is not None:
        _need(k_norm_weight, "k_norm_weight", torch.float32, shape=(HEAD_DIM,))
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16, shape=q.shape)
    _need(lse, "lse", torch.float32, shape=q.shape[:3])
    if workspace is None:
        workspace = torch.empty(prefill_workspace_size(plan, B, Sq, nnz), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8, 1)
    _check(load().pa_prefill(plan.handle, B, Sq, num_pages, nnz, _ptr(kv_indptr), _ptr(kv_indices),
                             _ptr(kv_last_page_len), _ptr(cache_position), _ptr(query_position_ids),
                             _ptr(key_position_ids), _ptr(q), _ptr(k_cache),
                             _ptr(v_cache), _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(out), _ptr(lse),
                             _ptr(workspace), int(workspace.numel()), _stream(stream)), "pa_prefill")
    return out, lse


def build_csr(block_table, kv_lens, kv_indptr=None, kv_indices=None, kv_last_page_len=None, stream=None):
    """pa_build_csr: CSR metadata from a dense block table on the device, without a host sync.

    block_table int32 [B, W] (-1 padded), kv_lens int32 [B].  Returns (kv_indptr [B+1],
    kv_indices [B*W], kv_last_page_len [B]), int32 device tensors (allocated here unless
    given).  The indices past kv_indptr[B] are -1; pass num_indices = B*W to decode/prefill."""
    import torch

    _need(block_table, "block_table", torch.int32, 2)
    B, W = (int(x) for x in block_table.shape)
    _need(kv_lens, "kv_lens", torch.int32, shape=(B,))
    dev = block_table.device
    if kv_indptr is None:
        kv_indptr = torch.empty(B + 1, dtype=torch.int32, device=dev)
    if kv_indices is None:
        kv_indices = torch.empty(max(B * W, 1), dtype=torch.int32, device=dev)
    if kv_last_page_len is None:
        kv_last_page_len = torch.empty(B, dtype=torch.int32, device=dev)
    _need(kv_indptr, "kv_indptr", torch.int32, shape=(B + 1,))
    _need(kv_indices, "kv_indices", torch.int32, 1)
    if kv_indices.numel() < B * W:
        raise ValueError(f"kv_indices holds {kv_indices.numel()} entries, need {B * W}")
    _need(kv_last_page_len, "kv_last_page_len", torch.int32, shape=(B,))
    _check(load().pa_build_csr(B, W, _ptr(block_table), _ptr(kv_lens), _ptr(kv_indptr), _ptr(kv_indices),
                               _ptr(kv_last_page_len), _stream(stream)), "pa_build_csr")
    return kv_indptr, kv_indices[:B * W], kv_last_page_len


def width_bucket(width: int) -> int:
    """pa_width_bucket: the power-of-two table width to make a plan for."""
    out = ctypes.c_int32()
    _check(load().pa_width_bucket(int(width), ctypes.byref(out)), "pa_width_bucket")
    return int(out.value)


def prefill_backward_workspace_size(plan: Plan, batch: int, seq_len: int) -> int:
    n = ctypes.c_size_t()
    _check(load().pa_prefill_backward_workspace_size(plan.handle, batch, seq_len, ctypes.byref(n)),
           "pa_prefill_backward_workspace_size")
    return int(n.value)


def prefill_backward(plan: Plan, positions, q, k, v, out, lse, dout, q_norm_weight=None, k_norm_weight=None,
                     workspace=None, stream=None, grads=None):
    """pa_prefill_backward on dense training-layout tensors.

    positions int32 [B, S]; q, out, dout bf16 [B, Hq, S, 128]; k, v bf16 [B, Hkv, S, 128];
    lse fp32 [B, Hq, S].  Returns (dq, dk, dv, dq_norm_weight, dk_norm_weight) as fp32 tensors
    (the weight gradients are None where that norm is absent).  ``grads``: optional tuple of
    those five tensors to write into instead of allocating them."""
    import torch

    _need(q, "q", torch.bfloat16, 4)
    B, Hq, S, D = q.shape
    if Hq != plan.num_q_heads or D != HEAD_DIM:
        raise ValueError(f"q shape {tuple(q.shape)} does not match the plan")
    kv_shape = (B, plan.num_kv_heads, S, D)
    _need(k, "k", torch.bfloat16, shape=kv_shape)
    _need(v, "v", torch.bfloat16, shape=kv_shape)
    _need(out, "out", torch.bfloat16, shape=q.shape)
    _need(dout, "dout", torch.bfloat16, shape=q.shape)
    _need(lse, "lse", torch.float32, shape=(B, Hq, S))
    _need(positions, "positions", torch.int32, shape=(B, S))
    for name, w in (("q_norm_weight", q_norm_weight), ("k_norm_weight", k_norm_weight)):
        if w is not None:
            _need(w, name, torch.float32, shape=(HEAD_DIM,))
    dev = q.device
    if grads is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
        dk = torch.empty(kv_shape, dtype=torch.float32, device=dev)
        dv = torch.empty(kv_shape, dtype=torch.float32, device=dev)
        dwq = torch.empty(HEAD_DIM, dtype=torch.float32, device=dev) if q_norm_weight is not None else None
        dwk = torch.empty(HEAD_DIM, dtype=torch.float32, device=dev) if k_norm_weight is not None else None
    else:
        dq, dk, dv, dwq, dwk = grads
        _need(dq, "dq", torch.float32, shape=q.shape)
        _need(dk, "dk", torch.float32, shape=kv_shape)
        _need(dv, "dv", torch.float32, shape=kv_shape)
        for name, g, w in (("dq_norm_weight", dwq, q_norm_weight), ("dk_norm_weight", dwk, k_norm_weight)):
            if w is not None:
                _need(g, name, torch.float32, shape=(HEAD_DIM,))
    if workspace is None:
        workspace = torch.empty(prefill_backward_workspace_size(plan, B, S), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, 1)
    _check(load().pa_prefill_backward(plan.handle, B, S, _ptr(positions), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(out), _ptr(lse), _ptr(dout),
                                      _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dwq), _ptr(dwk), _ptr(workspace),
                                      int(workspace.numel()), _stream(stream)), "pa_prefill_backward")
    return dq, dk, dv, dwq, dwk
