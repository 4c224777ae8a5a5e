"""MoBA (Mixture of Block Attention) prefill forward for MI355X (gfx950).

Python face of libmoba.so. PyTorch supplies device memory and the stream;
every step of the computation runs in the library's HIP kernels.

    o, idx = forward(q, k, v, block_size, top_k, causal=True)

q: [batch, heads, seq_len, head_dim]; k, v: [batch, kv_heads, seq_len,
head_dim] with heads a multiple of kv_heads (grouped-query attention; query
head h reads key/value head h // (heads // kv_heads)); contiguous CUDA
tensors, float32 or bfloat16. o has q's shape and dtype; idx is int32
[batch, heads, seq_len, top_k] with each query's chosen blocks ascending
(own block included), -1 padded. gate_shared=True routes the query heads of
one key/value head together, on the sum of their gate scores.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import (MOBA_BF16, MOBA_F32, moba_abi_version, moba_dense_causal_forward, moba_dense_forward,
                   moba_forward, moba_forward_lse, moba_last_error, moba_debug_pool, moba_problem_t,
                   moba_debug_gate_topk, moba_status_str,
                   moba_timing_enable, moba_timing_read, moba_workspace_size,
                   moba_forward_varlen, moba_forward_varlen_lse, moba_workspace_size_varlen, moba_backward,
                   moba_backward_workspace_size, moba_backward_varlen, moba_backward_workspace_size_varlen)

__all__ = ["MobaError", "forward", "dense", "pool", "select", "problem", "workspace_bytes",
           "timing", "moba_abi_version", "moba_forward", "moba_dense_causal_forward", "moba_dense_forward",
           "moba_debug_pool", "moba_debug_gate_topk", "moba_workspace_size", "moba_status_str", "moba_last_error",
           "moba_timing_enable", "moba_timing_read", "moba_problem_t"]

_DTYPES = {torch.float32: MOBA_F32, torch.bfloat16: MOBA_BF16}


class MobaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = _lib.STATUS_NAMES.get(status, str(status))
        super().__init__(f"{where}: {self.name} ({moba_status_str(status)}): {moba_last_error()}")


def _check(status: int, where: str):
    if status != 0:
        raise MobaError(status, where)


POOLINGS = {"mean": 0, "max": 1, "mean+max": 2}


def problem(q: torch.Tensor, block_size: int, top_k: int, causal: bool = True,
            pooling: str = "mean", kv_heads: int = 0, gate_shared: bool = False) -> moba_problem_t:
    if pooling not in POOLINGS:
        raise ValueError(f"pooling must be one of {tuple(POOLINGS)}, got {pooling!r}")
    if q.dim() != 4:
        raise ValueError(f"q must be [batch, heads, seq_len, head_dim], got shape {tuple(q.shape)}")
    if q.dtype not in _DTYPES:
        raise ValueError(f"dtype must be float32 or bfloat16, got {q.dtype}")
    B, H, S, D = q.shape
    return moba_problem_t(B, H, S, D, int(block_size), int(top_k), 1 if causal else 0, _DTYPES[q.dtype],
                          POOLINGS[pooling], 0, int(kv_heads), 1 if gate_shared else 0, 0)


def _tensors(q, *kv):
    """Checks q and the key/value tensors; returns kv_heads (0 if no k/v)."""
    for t in (q, *kv):
        if not t.is_cuda:
            raise ValueError("tensors must be on a GPU device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k and v must share dtype and device")
    if not kv:
        return 0
    k = kv[0]
    for t in kv:
        if t.dim() != 4 or t.shape != k.shape:
            raise ValueError("k and v must share one [batch, kv_heads, seq_len, head_dim] shape")
    if q.dim() != 4 or (k.shape[0], k.shape[2], k.shape[3]) != (q.shape[0], q.shape[2], q.shape[3]) \
            or k.shape[1] < 1 or q.shape[1] % k.shape[1]:
        raise ValueError(f"k, v {tuple(k.shape)} must be [batch, kv_heads, seq_len, head_dim] with heads a "
                         f"multiple of kv_heads, for q {tuple(q.shape)}")
    return int(k.shape[1])


def check_buffer(t, name: str, shape, dtype, device):
    """A caller-supplied output or input buffer must have exactly this shape,
    dtype and device and be contiguous: the kernels index it from those
    sizes, so a smaller or differently typed buffer would be read or written
    out of bounds. Returns t; raises ValueError naming the buffer."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != torch.device(device):
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def check_workspace(ws, need: int, device) -> int:
    """A caller-supplied workspace: a contiguous tensor on the device with at
    least `need` bytes. Returns its size in bytes (numel * element size)."""
    if not isinstance(ws, torch.Tensor):
        raise ValueError(f"workspace must be a tensor, got {type(ws).__name__}")
    if ws.device != torch.device(device):
        raise ValueError(f"workspace must be on {device}, got {ws.device}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    n = ws.numel() * ws.element_size()
    if n < need:
        raise ValueError(f"workspace holds {n} bytes, the problem needs {need}")
    return n


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def workspace_bytes(p: moba_problem_t) -> int:
    st, n = moba_workspace_size(p)
    _check(st, "moba_workspace_size")
    return n


def _workspace(p, device):
    n = workspace_bytes(p)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=device)
    if ws.data_ptr() % 256:
        raise RuntimeError("workspace allocation is not 256-byte aligned")
    return ws, n


def forward(q, k, v, block_size: int, top_k: int, causal: bool = True, out=None, idx=None,
            workspace=None, pooling: str = "mean", gate_shared: bool = False, return_lse: bool = False):
    """MoBA forward. Returns (o, block_idx), or (o, block_idx, lse) with
    return_lse (float32 [B, H, S], the natural-log log-sum-exp of each
    query's scaled logits over its attended keys). pooling: the gate's
    block summary, "mean" (the paper's), "max" or "mean+max". gate_shared:
    the query heads of one key/value head route on their summed scores."""
    hkv = _tensors(q, k, v)
    p = problem(q, block_size, top_k, causal, pooling, hkv, gate_shared)
    B, H, S, D = q.shape
    need = workspace_bytes(p)  # validates the problem through the library first
    o = torch.empty_like(q) if out is None else check_buffer(out, "out", q.shape, q.dtype, q.device)
    idx_shape = (B, H, S, int(top_k))
    bi = torch.empty(idx_shape, dtype=torch.int32, device=q.device) if idx is None else \
        check_buffer(idx, "idx", idx_shape, torch.int32, q.device)
    if workspace is None:
        ws, n = _workspace(p, q.device)
    else:
        ws, n = workspace, check_workspace(workspace, need, q.device)
    with torch.cuda.device(q.device):
        if return_lse:
            lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
            _check(moba_forward_lse(p, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), bi.data_ptr(),
                                    lse.data_ptr(), ws.data_ptr(), n, _stream(q.device)), "moba_forward_lse")
            return o, bi, lse
        _check(moba_forward(p, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), bi.data_ptr(),
                            ws.data_ptr(), n, _stream(q.device)), "moba_forward")
    return o, bi


def backward(q, k, v, o, dout, idx, lse, block_size: int, top_k: int, causal: bool = True):
    """MoBA backward (bf16): (dq, dk, dv) for the upstream gradient dout,
    with the forward's block choice idx held fixed; o and lse from
    forward(..., return_lse=True)."""
    hkv = _tensors(q, k, v)
    _tensors(q, o, dout)
    p = problem(q, block_size, top_k, causal, "mean", hkv)
    st, n = moba_backward_workspace_size(p)  # validates the problem through the library first
    _check(st, "moba_backward_workspace_size")
    check_buffer(o, "o", q.shape, q.dtype, q.device)
    check_buffer(dout, "dout", q.shape, q.dtype, q.device)
    B, H, S, D = q.shape
    check_buffer(idx, "idx", (B, H, S, int(top_k)), torch.int32, q.device)
    check_buffer(lse, "lse", (B, H, S), torch.float32, q.device)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    with torch.cuda.device(q.device):
        _check(moba_backward(p, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                             idx.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                             ws.data_ptr(), n, _stream(q.device)), "moba_backward")
    return dq, dk, dv


def forward_varlen(q, k, v, cu_seqlens, heads: int, block_size: int, top_k: int, causal: bool = True,
                   pooling: str = "mean", kv_heads: int = 0, gate_shared: bool = False, return_lse: bool = False):
    """MoBA over a varlen batch: sequences of different lengths (any length
    >= 1) back to back, run as one launch chain.

    q: [sum_i heads * len_i, head_dim], sequence i's [heads, len_i, head_dim]
    rows from row cu_seqlens[i] * heads (see pack_varlen); k, v likewise
    with kv_heads (0 = heads). cu_seqlens: host ints, cu_seqlens[0] = 0.
    Returns (o like q, block_idx int32 [sum_i heads * len_i, top_k] in the
    same order), and with return_lse also lse float32 [sum_i heads * len_i]
    (each query's natural-log log-sum-exp, for backward_varlen)."""
    if q.dim() != 2:
        raise ValueError(f"q must be [tokens * heads, head_dim], got shape {tuple(q.shape)}")
    hkv = int(kv_heads) or int(heads)
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 2 or t.shape[1] != q.shape[1] \
                or t.dtype != q.dtype:
            raise ValueError("q, k and v must be contiguous 2-D GPU tensors of one head_dim and dtype")
    if k.shape != v.shape or k.shape[0] * heads != q.shape[0] * hkv:
        raise ValueError(f"k, v {tuple(k.shape)} must hold kv_heads={hkv} rows per token of q {tuple(q.shape)}")
    if q.dtype not in _DTYPES:
        raise ValueError(f"dtype must be float32 or bfloat16, got {q.dtype}")
    if pooling not in POOLINGS:
        raise ValueError(f"pooling must be one of {tuple(POOLINGS)}, got {pooling!r}")
    cu = [int(x) for x in cu_seqlens]
    if q.shape[0] != cu[-1] * heads:
        raise ValueError(f"q has {q.shape[0]} rows, cu_seqlens and heads give {cu[-1] * heads}")
    p = moba_problem_t(len(cu) - 1, int(heads), cu[-1], q.shape[1], int(block_size), int(top_k),
                       1 if causal else 0, _DTYPES[q.dtype], POOLINGS[pooling], 0, int(kv_heads),
                       1 if gate_shared else 0, 0)
    st, n = moba_workspace_size_varlen(p, cu)
    _check(st, "moba_workspace_size_varlen")
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    bi = torch.empty((q.shape[0], int(top_k)), dtype=torch.int32, device=q.device)
    with torch.cuda.device(q.device):
        if return_lse:
            lse = torch.empty(q.shape[0], dtype=torch.float32, device=q.device)
            _check(moba_forward_varlen_lse(p, cu, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                           bi.data_ptr(), lse.data_ptr(), ws.data_ptr(), n, _stream(q.device)),
                   "moba_forward_varlen_lse")
            return o, bi, lse
        _check(moba_forward_varlen(p, cu, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), bi.data_ptr(),
                                   ws.data_ptr(), n, _stream(q.device)), "moba_forward_varlen")
    return o, bi


def backward_varlen(q, k, v, o, dout, idx, lse, cu_seqlens, heads: int, block_size: int, top_k: int,
                    causal: bool = True, kv_heads: int = 0, gate_shared: bool = False):
    """MoBA backward (bf16) of a varlen batch laid out as forward_varlen's:
    (dq like q, dk like k, dv like v), each sequence's gradients as
    backward computes them for that sequence alone; idx and lse from
    forward_varlen(..., return_lse=True) on the same batch."""
    if q.dim() != 2:
        raise ValueError(f"q must be [tokens * heads, head_dim], got shape {tuple(q.shape)}")
    for t in (q, k, v, o, dout):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 2 or t.shape[1] != q.shape[1] \
                or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v, o and dout must be contiguous 2-D tensors on one GPU, of one head_dim and dtype")
    if q.dtype not in _DTYPES:
        raise ValueError(f"dtype must be float32 or bfloat16, got {q.dtype}")
    hkv = int(kv_heads) or int(heads)
    if o.shape != q.shape or dout.shape != q.shape or k.shape != v.shape or k.shape[0] * heads != q.shape[0] * hkv:
        raise ValueError("o and dout must be shaped like q, and k, v must hold kv_heads rows per token of q")
    cu = [int(x) for x in cu_seqlens]
    if q.shape[0] != cu[-1] * heads:
        raise ValueError(f"q has {q.shape[0]} rows, cu_seqlens and heads give {cu[-1] * heads}")
    p = moba_problem_t(len(cu) - 1, int(heads), cu[-1], q.shape[1], int(block_size), int(top_k),
                       1 if causal else 0, _DTYPES[q.dtype], 0, 0, int(kv_heads), 1 if gate_shared else 0, 0)
    st, n = moba_backward_workspace_size_varlen(p, cu)  # validates every sequence through the library first
    _check(st, "moba_backward_workspace_size_varlen")
    check_buffer(idx, "idx", (q.shape[0], int(top_k)), torch.int32, q.device)
    check_buffer(lse, "lse", (q.shape[0],), torch.float32, q.device)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    with torch.cuda.device(q.device):
        _check(moba_backward_varlen(p, cu, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                    idx.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                    ws.data_ptr(), n, _stream(q.device)), "moba_backward_varlen")
    return dq, dk, dv


def pack_varlen(seqs):
    """[1, heads, len_i, D] tensors -> ([sum heads * len_i, D], cu_seqlens)."""
    cu = [0]
    for x in seqs:
        cu.append(cu[-1] + x.shape[2])
    return torch.cat([x.reshape(-1, x.shape[3]) for x in seqs]), cu


def unpack_varlen(x, cu_seqlens, heads: int):
    """Inverse of pack_varlen for an output (o or block_idx) of forward_varlen."""
    return [x[cu_seqlens[i] * heads:cu_seqlens[i + 1] * heads].reshape(1, heads, cu_seqlens[i + 1] - cu_seqlens[i], -1)
            for i in range(len(cu_seqlens) - 1)]


def dense(q, k, v, causal: bool = True, out=None):
    """Full softmax attention (causal or not) with the library's dense
    kernel: moba_dense_causal_forward, or moba_dense_forward without the
    causal mask."""
    hkv = _tensors(q, k, v)
    p = problem(q, q.shape[2], 1, causal, kv_heads=hkv)
    o = torch.empty_like(q) if out is None else check_buffer(out, "out", q.shape, q.dtype, q.device)
    fn, name = (moba_dense_causal_forward, "moba_dense_causal_forward") if causal else \
        (moba_dense_forward, "moba_dense_forward")
    with torch.cuda.device(q.device):
        _check(fn(p, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _stream(q.device)), name)
    return o


def pool(k, block_size: int, pooling: str = "mean"):
    """Block summaries of K as the gate uses them: float64 [B, H, n_blocks, D]."""
    _tensors(k)
    p = problem(k, block_size, 1, True, pooling)
    B, H, S, D = k.shape
    nb = -(-S // block_size) if block_size > 0 else 0  # a short last block counts
    kbar = torch.empty((B, H, nb, D), dtype=torch.float64, device=k.device)
    ws, n = _workspace(p, k.device)
    with torch.cuda.device(k.device):
        _check(moba_debug_pool(p, k.data_ptr(), kbar.data_ptr(), ws.data_ptr(), n, _stream(k.device)),
               "moba_debug_pool")
    return kbar


def select(q, k, block_size: int, top_k: int, causal: bool = True, pooling: str = "mean",
           gate_shared: bool = False):
    """Routing only: int32 [B, H, S, top_k] exactly as forward() returns it."""
    hkv = _tensors(q, k)
    p = problem(q, block_size, top_k, causal, pooling, hkv, gate_shared)
    B, H, S, D = q.shape
    bi = torch.empty((B, H, S, int(top_k)), dtype=torch.int32, device=q.device)
    ws, n = _workspace(p, q.device)
    with torch.cuda.device(q.device):
        _check(moba_debug_gate_topk(p, q.data_ptr(), k.data_ptr(), bi.data_ptr(), ws.data_ptr(), n,
                                    _stream(q.device)), "moba_debug_gate_topk")
    return bi


class timing:
    """Context manager: per-kernel HIP-event timing of library launches.

        with timing() as t: ...
        t.rows -> [(kernel, launches, total_ms), ...]
    """

    def __enter__(self):
        _check(moba_timing_enable(True), "moba_timing_enable")
        moba_timing_read()  # drop anything recorded before
        self.rows = []
        return self

    def __exit__(self, *exc):
        _check(moba_timing_enable(False), "moba_timing_enable")
        st, self.rows = moba_timing_read(64)
        _check(st, "moba_timing_read")
        return False
