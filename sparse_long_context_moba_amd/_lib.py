"""ctypes declarations of libmoba.so's C ABI (include/moba.h), same names.

Argument marshalling only: every step of the MoBA forward runs in the HIP
kernels behind these entry points. There is no fallback: if libmoba.so is
missing or fails to load, the first call (or lib()) raises ImportError. The
library is opened on first use so that the build module can be imported
before anything is built.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoba.so")

MOBA_F32, MOBA_BF16 = 0, 1
STATUS_NAMES = {0: "MOBA_OK", 1: "MOBA_ERR_NULL", 2: "MOBA_ERR_SHAPE", 3: "MOBA_ERR_ARG",
                4: "MOBA_ERR_DTYPE", 5: "MOBA_ERR_UNSUPPORTED", 6: "MOBA_ERR_WORKSPACE",
                7: "MOBA_ERR_DEVICE"}
EXPORTED = ["moba_abi_version", "moba_status_str", "moba_last_error", "moba_workspace_size",
            "moba_forward", "moba_forward_noalloc", "moba_forward_lse", "moba_dense_causal_forward", "moba_dense_forward",
            "moba_debug_pool", "moba_debug_gate_topk",
            "moba_workspace_size_varlen", "moba_forward_varlen", "moba_forward_varlen_lse",
            "moba_backward_workspace_size", "moba_backward",
            "moba_backward_workspace_size_varlen", "moba_backward_varlen",
            "moba_timing_enable", "moba_timing_read"]


class moba_problem_t(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("heads", ctypes.c_int64), ("seq_len", ctypes.c_int64),
                ("head_dim", ctypes.c_int64), ("block_size", ctypes.c_int64),
                ("top_k", ctypes.c_int64), ("causal", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("pooling", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("kv_heads", ctypes.c_int64), ("gate_shared", ctypes.c_int32), ("reserved2", ctypes.c_int32)]


class moba_kernel_time_t(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m sparse_long_context_moba_amd.build` "
                          "(hipcc, gfx950). There is no non-HIP fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(moba_problem_t)
    vp, sz, i32p = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p
    sig = {
        "moba_abi_version": ([], ctypes.c_int),
        "moba_status_str": ([ctypes.c_int], ctypes.c_char_p),
        "moba_last_error": ([], ctypes.c_char_p),
        "moba_workspace_size": ([P, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
        "moba_forward": ([P, vp, vp, vp, vp, i32p, vp, sz, vp], ctypes.c_int),
        "moba_forward_noalloc": ([P, vp, vp, vp, vp, i32p, vp], ctypes.c_int),
        "moba_forward_lse": ([P, vp, vp, vp, vp, i32p, vp, vp, sz, vp], ctypes.c_int),
        "moba_dense_causal_forward": ([P, vp, vp, vp, vp, vp], ctypes.c_int),
        "moba_dense_forward": ([P, vp, vp, vp, vp, vp], ctypes.c_int),
        "moba_debug_pool": ([P, vp, vp, vp, sz, vp], ctypes.c_int),
        "moba_debug_gate_topk": ([P, vp, vp, i32p, vp, sz, vp], ctypes.c_int),
        "moba_workspace_size_varlen": ([P, ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
                                        ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
        "moba_forward_varlen": ([P, ctypes.POINTER(ctypes.c_int64), ctypes.c_int64, vp, vp, vp, vp, i32p, vp,
                                 sz, vp], ctypes.c_int),
        "moba_forward_varlen_lse": ([P, ctypes.POINTER(ctypes.c_int64), ctypes.c_int64, vp, vp, vp, vp, i32p, vp,
                                     vp, sz, vp], ctypes.c_int),
        "moba_backward_workspace_size": ([P, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
        "moba_backward": ([P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "moba_backward_workspace_size_varlen": ([P, ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
                                                 ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
        "moba_backward_varlen": ([P, ctypes.POINTER(ctypes.c_int64), ctypes.c_int64, vp, vp, vp, vp, vp, vp, vp,
                                  vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "moba_timing_enable": ([ctypes.c_int], ctypes.c_int),
        "moba_timing_read": ([ctypes.POINTER(moba_kernel_time_t), ctypes.c_int,
                              ctypes.POINTER(ctypes.c_int)], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_LIB = None


def lib():
    """The loaded libmoba.so (opened on first use; raises if not built)."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def moba_abi_version() -> int:
    return lib().moba_abi_version()


def moba_status_str(status: int) -> str:
    return lib().moba_status_str(status).decode()


def moba_last_error() -> str:
    return lib().moba_last_error().decode()


def moba_workspace_size(problem: moba_problem_t):
    """-> (status, bytes)"""
    n = ctypes.c_size_t(0)
    st = lib().moba_workspace_size(ctypes.byref(problem) if problem is not None else None, ctypes.byref(n))
    return st, n.value


def moba_forward(problem, q, k, v, o, block_idx, workspace, workspace_bytes, stream) -> int:
    return lib().moba_forward(ctypes.byref(problem) if problem is not None else None,
                            q, k, v, o, block_idx, workspace, workspace_bytes, stream)


def moba_forward_noalloc(problem, q, k, v, o, block_idx, stream) -> int:
    return lib().moba_forward_noalloc(ctypes.byref(problem) if problem is not None else None,
                                      q, k, v, o, block_idx, stream)


NOALLOC_SCRATCH_BYTES = 256 << 20  # MOBA_NOALLOC_SCRATCH_BYTES in include/moba.h


def moba_forward_lse(problem, q, k, v, o, block_idx, lse, workspace, workspace_bytes, stream) -> int:
    return lib().moba_forward_lse(ctypes.byref(problem) if problem is not None else None,
                                  q, k, v, o, block_idx, lse, workspace, workspace_bytes, stream)


def _cu(cu_seqlens):
    """Host int64 array for cu_seqlens (None stays NULL)."""
    if cu_seqlens is None:
        return None, 0
    arr = (ctypes.c_int64 * len(cu_seqlens))(*[int(x) for x in cu_seqlens])
    return arr, len(cu_seqlens) - 1


def moba_workspace_size_varlen(problem, cu_seqlens, n_seqs=None):
    """-> (status, bytes); n_seqs defaults to len(cu_seqlens) - 1."""
    arr, n = _cu(cu_seqlens)
    out = ctypes.c_size_t(0)
    st = lib().moba_workspace_size_varlen(ctypes.byref(problem) if problem is not None else None, arr,
                                          n if n_seqs is None else n_seqs, ctypes.byref(out))
    return st, out.value


def moba_forward_varlen(problem, cu_seqlens, q, k, v, o, block_idx, workspace, workspace_bytes, stream,
                        n_seqs=None) -> int:
    arr, n = _cu(cu_seqlens)
    return lib().moba_forward_varlen(ctypes.byref(problem) if problem is not None else None, arr,
                                     n if n_seqs is None else n_seqs, q, k, v, o, block_idx, workspace,
                                     workspace_bytes, stream)


def moba_forward_varlen_lse(problem, cu_seqlens, q, k, v, o, block_idx, lse, workspace, workspace_bytes, stream,
                            n_seqs=None) -> int:
    arr, n = _cu(cu_seqlens)
    return lib().moba_forward_varlen_lse(ctypes.byref(problem) if problem is not None else None, arr,
                                         n if n_seqs is None else n_seqs, q, k, v, o, block_idx, lse, workspace,
                                         workspace_bytes, stream)


def moba_backward_workspace_size_varlen(problem, cu_seqlens, n_seqs=None):
    """-> (status, bytes); n_seqs defaults to len(cu_seqlens) - 1."""
    arr, n = _cu(cu_seqlens)
    out = ctypes.c_size_t(0)
    st = lib().moba_backward_workspace_size_varlen(ctypes.byref(problem) if problem is not None else None, arr,
                                                   n if n_seqs is None else n_seqs, ctypes.byref(out))
    return st, out.value


def moba_backward_varlen(problem, cu_seqlens, q, k, v, o, dout, block_idx, lse, dq, dk, dv, workspace,
                         workspace_bytes, stream, n_seqs=None) -> int:
    arr, n = _cu(cu_seqlens)
    return lib().moba_backward_varlen(ctypes.byref(problem) if problem is not None else None, arr,
                                      n if n_seqs is None else n_seqs, q, k, v, o, dout, block_idx, lse, dq, dk,
                                      dv, workspace, workspace_bytes, stream)


def moba_dense_causal_forward(problem, q, k, v, o, stream) -> int:
    return lib().moba_dense_causal_forward(ctypes.byref(problem) if problem is not None else None, q, k, v, o,
                                           stream)


def moba_dense_forward(problem, q, k, v, o, stream) -> int:
    return lib().moba_dense_forward(ctypes.byref(problem) if problem is not None else None, q, k, v, o, stream)


def moba_debug_pool(problem, k, kbar, workspace, workspace_bytes, stream) -> int:
    return lib().moba_debug_pool(ctypes.byref(problem) if problem is not None else None, k, kbar, workspace,
                                 workspace_bytes, stream)


def moba_debug_gate_topk(problem, q, k, block_idx, workspace, workspace_bytes, stream) -> int:
    return lib().moba_debug_gate_topk(ctypes.byref(problem) if problem is not None else None, q, k, block_idx,
                                      workspace, workspace_bytes, stream)


def moba_backward_workspace_size(problem):
    """-> (status, bytes)"""
    n = ctypes.c_size_t(0)
    st = lib().moba_backward_workspace_size(ctypes.byref(problem) if problem is not None else None, ctypes.byref(n))
    return st, n.value


def moba_backward(problem, q, k, v, o, dout, block_idx, lse, dq, dk, dv, workspace, workspace_bytes, stream) -> int:
    return lib().moba_backward(ctypes.byref(problem) if problem is not None else None, q, k, v, o, dout, block_idx,
                               lse, dq, dk, dv, workspace, workspace_bytes, stream)


def moba_timing_enable(enable: bool) -> int:
    return lib().moba_timing_enable(1 if enable else 0)


def moba_timing_read(max_entries: int = 32):
    """-> (status, [(name, launches, total_ms), ...])"""
    buf = (moba_kernel_time_t * max_entries)()
    n = ctypes.c_int(0)
    st = lib().moba_timing_read(buf, max_entries, ctypes.byref(n))
    rows = [(buf[i].name.decode(), int(buf[i].launches), float(buf[i].total_ms))
            for i in range(min(n.value, max_entries))]
    return st, rows
