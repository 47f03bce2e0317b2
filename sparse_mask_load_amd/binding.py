"""Thin ctypes binding of libsparse_attn.so (argument marshalling only).

Every computation runs in the library's HIP kernels; PyTorch only supplies device
memory (``tensor.data_ptr()``) and the current HIP stream.  The functions carry the
names of the C entry points declared in ``include/sparse_attn.h``.  If the shared
library has not been built, every call raises instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_attn.so")

SA_OK, SA_ERR_INVALID, SA_ERR_UNSUPPORTED, SA_ERR_HIP, SA_ERR_NOMEM = 0, -1, -2, -3, -4
SA_F32, SA_BF16 = 0, 1
SA_ORDER_LPT, SA_ORDER_NAIVE, SA_ORDER_LPT_XCD, SA_ORDER_LPT_DEVICE, SA_ORDER_LPT_DYNAMIC = 0, 1, 2, 3, 4
SA_LAYOUT_CONTIGUOUS, SA_LAYOUT_STRIPED = 0, 1
SA_KIND_BLOCK, SA_KIND_TOPK, SA_KIND_INDEX = 0, 1, 2
(SA_PLAN_ROW, SA_PLAN_COL, SA_PLAN_CROW, SA_PLAN_ITEMS, SA_PLAN_BIN_PTR, SA_PLAN_BIN_LOAD,
 SA_PLAN_TOPK_IDX, SA_PLAN_TOPK_COUNT, SA_PLAN_PAIR_ROW, SA_PLAN_PAIR_CROW, SA_PLAN_LPT_ORDER) = range(11)

_DTYPES = {"f32": SA_F32, "bf16": SA_BF16}
_ORDERS = {"lpt": SA_ORDER_LPT, "naive": SA_ORDER_NAIVE, "lpt_xcd": SA_ORDER_LPT_XCD,
           "lpt_device": SA_ORDER_LPT_DEVICE, "lpt_dynamic": SA_ORDER_LPT_DYNAMIC}
_LAYOUTS = {"contiguous": SA_LAYOUT_CONTIGUOUS, "striped": SA_LAYOUT_STRIPED}


class SparseAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class sa_problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("S", ctypes.c_int32), ("D", ctypes.c_int32),
                ("block", ctypes.c_int32), ("n_chunks", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("token_causal", ctypes.c_int32),
                ("q_pairs", ctypes.c_int32), ("sb", ctypes.c_int64), ("sh", ctypes.c_int64),
                ("ss", ctypes.c_int64)]


class sa_sparsity(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("rank", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("mask", ctypes.c_void_p), ("q", ctypes.c_void_p),
                ("k", ctypes.c_void_p), ("wq", ctypes.c_void_p), ("wk", ctypes.c_void_p),
                ("idx", ctypes.c_void_p), ("count", ctypes.c_void_p)]


class sa_plan_info(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("num_bins", ctypes.c_int32), ("order", ctypes.c_int32),
                ("n_chunks", ctypes.c_int32), ("nQ", ctypes.c_int32), ("nK", ctypes.c_int32),
                ("n_items", ctypes.c_int32), ("top_k", ctypes.c_int32), ("total_live", ctypes.c_int64),
                ("load_sum", ctypes.c_int64), ("makespan", ctypes.c_int64), ("lower_bound", ctypes.c_int64),
                ("groups", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_P = ctypes.c_void_p
_SIGNATURES = {
    "sparse_attn_plan": (ctypes.c_int32, [ctypes.POINTER(sa_problem), ctypes.POINTER(sa_sparsity), ctypes.c_int32,
                                          ctypes.c_int32, ctypes.POINTER(_P), _P]),
    "sparse_attn_fwd": (ctypes.c_int32, [_P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P, _P]),
    "sparse_attn_fwd_noalloc": (ctypes.c_int32, [ctypes.POINTER(sa_problem), _P, ctypes.c_int32, _P, _P, _P,
                                                 ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P]),
    "chunk_merge": (ctypes.c_int32, [ctypes.c_int32, ctypes.POINTER(_P), ctypes.POINTER(_P), ctypes.POINTER(_P),
                                     ctypes.c_int64, ctypes.c_int32, _P, ctypes.c_int32, _P, _P]),
    "sparse_attn_plan_info": (ctypes.c_int32, [_P, ctypes.POINTER(sa_plan_info)]),
    "sparse_attn_plan_copy": (ctypes.c_int32, [_P, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int64]),
    "sparse_attn_assign_host": (ctypes.c_int32, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
    "sparse_attn_assign_host_grouped": (ctypes.c_int32, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                         ctypes.c_int32, _P, _P, _P]),
    "sparse_attn_plan_destroy": (None, [_P]),
    "sa_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "sa_last_error": (ctypes.c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libsparse_attn.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m sparse_mask_load_amd.build` "
                               "(or __graft_entry__.build()) first")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def sa_status_string(status: int) -> str:
    return lib().sa_status_string(status).decode()


def sa_last_error() -> str:
    return lib().sa_last_error().decode()


def _check(status: int, what: str) -> None:
    if status != SA_OK:
        raise SparseAttnError(status, f"{what}: {sa_status_string(status)}: {sa_last_error()}")


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(getattr(stream, "cuda_stream", stream))  # a torch stream or a raw handle
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def make_problem(q, block: int = 0, n_chunks: int = 1, layout: str = "contiguous",
                 scale: float = 0.0, token_causal: bool = False, q_pairs: bool = False) -> sa_problem:
    """Describe a [B, H, S, D] tensor (last dim contiguous) as an sa_problem."""
    import torch
    if q.dim() != 4 or q.stride(-1) != 1:
        raise ValueError("q must be [B, H, S, D] with a contiguous last dimension")
    dtype = {torch.bfloat16: SA_BF16, torch.float32: SA_F32}[q.dtype]
    B, H, S, D = q.shape
    return sa_problem(B, H, S, D, block, n_chunks, _LAYOUTS[layout], dtype, float(scale), 1 if token_causal else 0,
                      1 if q_pairs else 0, q.stride(0), q.stride(1), q.stride(2))


class Plan:
    """Owns an sa_plan*; freed by sparse_attn_plan_destroy on close() / garbage collection."""

    def __init__(self, handle: int, problem: sa_problem):
        self.handle = handle
        self.problem = problem

    def close(self) -> None:
        if self.handle:
            lib().sparse_attn_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def sparse_attn_plan(problem: sa_problem, kind: str = "block", mask=None, q=None, k=None, wq=None, wk=None,
                     idx=None, count=None, rank: int = 32, top_k: int = 0, causal: bool = True,
                     num_bins: int = 0, order: str = "lpt", stream=None) -> Plan:
    sp = sa_sparsity({"block": SA_KIND_BLOCK, "topk": SA_KIND_TOPK, "index": SA_KIND_INDEX}[kind], rank, top_k,
                     1 if causal else 0, _ptr(mask), _ptr(q), _ptr(k), _ptr(wq), _ptr(wk), _ptr(idx), _ptr(count))
    out = _P()
    _check(lib().sparse_attn_plan(ctypes.byref(problem), ctypes.byref(sp), num_bins, _ORDERS[order],
                                  ctypes.byref(out), _stream(stream)), "sparse_attn_plan")
    return Plan(out.value, problem)


def sparse_attn_fwd(plan: Plan, q, k, v, chunk_begin: int = 0, chunk_end: Optional[int] = None, o=None,
                    o_part=None, m_part=None, l_part=None, trace=None, stream=None) -> None:
    if chunk_end is None:
        chunk_end = max(1, plan.problem.n_chunks)
    _check(lib().sparse_attn_fwd(plan.handle, _ptr(q), _ptr(k), _ptr(v), chunk_begin, chunk_end, _ptr(o),
                                 _ptr(o_part), _ptr(m_part), _ptr(l_part), _ptr(trace), _stream(stream)),
           "sparse_attn_fwd")


def sparse_attn_fwd_noalloc(problem: sa_problem, mask, q, k, v, chunk_begin: int = 0,
                            chunk_end: Optional[int] = None, o=None, o_part=None, m_part=None, l_part=None,
                            num_bins: int = 0, stream=None) -> None:
    if chunk_end is None:
        chunk_end = max(1, problem.n_chunks)
    _check(lib().sparse_attn_fwd_noalloc(ctypes.byref(problem), _ptr(mask), num_bins, _ptr(q), _ptr(k), _ptr(v),
                                         chunk_begin, chunk_end, _ptr(o), _ptr(o_part), _ptr(m_part),
                                         _ptr(l_part), _stream(stream)), "sparse_attn_fwd_noalloc")


def chunk_merge(o_parts: Sequence, m_parts: Sequence, l_parts: Sequence, rows: int, D: int, o_out,
                out_dtype: str = "bf16", lse_out=None, stream=None) -> None:
    n = len(o_parts)
    arr = _P * max(n, 1)
    po = arr(*[_ptr(t) for t in o_parts])
    pm = arr(*[_ptr(t) for t in m_parts])
    pl = arr(*[_ptr(t) for t in l_parts])
    _check(lib().chunk_merge(n, po, pm, pl, rows, D, _ptr(o_out), _DTYPES[out_dtype], _ptr(lse_out),
                             _stream(stream)), "chunk_merge")


def sparse_attn_plan_info(plan: Plan) -> dict:
    info = sa_plan_info()
    _check(lib().sparse_attn_plan_info(plan.handle, ctypes.byref(info)), "sparse_attn_plan_info")
    return {name: getattr(info, name) for name, _ in sa_plan_info._fields_}


_COPY_SHAPES = {SA_PLAN_BIN_LOAD: np.int64}


def sparse_attn_plan_copy(plan: Plan, what: int, n_elems: int, chunk: int = -1) -> np.ndarray:
    out = np.empty(n_elems, dtype=_COPY_SHAPES.get(what, np.int32))
    _check(lib().sparse_attn_plan_copy(plan.handle, what, chunk, out.ctypes.data, n_elems), "sparse_attn_plan_copy")
    return out


def sparse_attn_assign_host(loads, m: int, order: str = "lpt"):
    loads = np.ascontiguousarray(loads, dtype=np.int64)
    n = loads.shape[0]
    items = np.empty(max(n, 1), np.int32)
    ptr = np.empty(m + 1, np.int32)
    bl = np.empty(m, np.int64)
    _check(lib().sparse_attn_assign_host(loads.ctypes.data, n, m, _ORDERS[order], items.ctypes.data,
                                         ptr.ctypes.data, bl.ctypes.data), "sparse_attn_assign_host")
    return items[:n], ptr, bl


def sparse_attn_assign_host_grouped(loads, items_per_head: int, m: int, groups: int):
    loads = np.ascontiguousarray(loads, dtype=np.int64).reshape(-1)
    n = loads.shape[0]
    items = np.empty(max(n, 1), np.int32)
    ptr = np.empty(m + 1, np.int32)
    bl = np.empty(m, np.int64)
    _check(lib().sparse_attn_assign_host_grouped(loads.ctypes.data, n // items_per_head, items_per_head, m, groups,
                                                 items.ctypes.data, ptr.ctypes.data, bl.ctypes.data),
           "sparse_attn_assign_host_grouped")
    return items[:n], ptr, bl


def sparse_attn_plan_destroy(plan: Plan) -> None:
    plan.close()
