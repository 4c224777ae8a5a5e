"""The C ABI without a GPU: the library loads, exports every function that
include/moba.h declares, and rejects bad arguments on the host (validation
happens before any HIP call, so these run anywhere)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "sparse_long_context_moba_amd", "libmoba.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmoba.so not built")


def _header_functions():
    text = open(os.path.join(ROOT, "include", "moba.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moba_\w+)\s*\(", text)))


def test_exports_every_declared_function():
    from sparse_long_context_moba_amd import _lib
    names = _header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(_lib.lib(), n), n
    assert sorted(_lib.EXPORTED) == names


# The boundary's entry points: the forward with its workspace query, the
# dense causal baseline, the two stage (debug) entry points and the status
# text; each must be declared in include/moba.h and exported by the library.
BOUNDARY = ["moba_abi_version", "moba_workspace_size", "moba_forward", "moba_dense_causal_forward",
            "moba_status_str", "moba_debug_pool", "moba_debug_gate_topk"]


def test_boundary_entry_points_are_declared_and_exported():
    from sparse_long_context_moba_amd import _lib
    names = _header_functions()
    for n in BOUNDARY:
        assert n in names, f"{n} not declared in include/moba.h"
        fn = getattr(_lib.lib(), n)
        assert fn is not None


def test_boundary_entry_points_validate_through_ctypes():
    """Each boundary entry point, called through ctypes with a bad argument,
    returns its status code before any launch."""
    from sparse_long_context_moba_amd import _lib
    st, need = _lib.moba_workspace_size(_p())
    assert st == 0
    assert _lib.moba_dense_causal_forward(_p(), None, FAKE, FAKE, FAKE, None) == 1
    assert _lib.moba_dense_causal_forward(_p(head_dim=96), FAKE, FAKE, FAKE, FAKE, None) == 5
    assert "head_dim" in _lib.moba_last_error()
    # p->causal does not matter to the causal baseline: still validated the same way
    assert _lib.moba_dense_causal_forward(_p(causal=0, dtype=9), FAKE, FAKE, FAKE, FAKE, None) == 4
    assert _lib.moba_debug_pool(_p(), None, FAKE, FAKE, need, None) == 1
    assert _lib.moba_debug_pool(_p(top_k=0), FAKE, FAKE, FAKE, need, None) == 3
    assert _lib.moba_debug_pool(_p(), FAKE, FAKE, FAKE, need - 1, None) == 6
    assert _lib.moba_debug_gate_topk(_p(), FAKE, None, FAKE, FAKE, need, None) == 1
    assert _lib.moba_debug_gate_topk(_p(block_size=96), FAKE, FAKE, FAKE, FAKE, need, None) == 5
    assert _lib.moba_debug_gate_topk(_p(), FAKE, FAKE, FAKE, None, need, None) == 6
    assert _lib.moba_status_str(0) == "ok"


def test_abi_version_and_status_strings():
    from sparse_long_context_moba_amd import _lib
    assert _lib.moba_abi_version() == 7
    for code in range(8):
        assert _lib.moba_status_str(code)
    assert _lib.moba_status_str(99) == "unknown status"


def _p(**kw):
    from sparse_long_context_moba_amd._lib import moba_problem_t
    base = dict(batch=1, heads=2, seq_len=1024, head_dim=128, block_size=256, top_k=3, causal=1, dtype=1)
    base.update(kw)
    return moba_problem_t(**base)


FAKE = 0x1000  # never dereferenced: validation fails or stops before any launch


@pytest.mark.parametrize("kw,code,word", [
    (dict(batch=0), 2, "batch"),
    (dict(heads=-1), 2, "heads"),
    (dict(seq_len=0), 2, "seq_len"),
    (dict(head_dim=0), 2, "head_dim"),
    (dict(block_size=0), 2, "block_size"),
    (dict(top_k=0), 3, "top_k"),
    (dict(pooling=3), 3, "pooling"),
    (dict(pooling=-1), 3, "pooling"),
    (dict(reserved=1), 3, "reserved"),
    (dict(reserved2=1), 3, "reserved2"),
    (dict(kv_heads=-1), 2, "kv_heads"),
    (dict(heads=4, kv_heads=3), 2, "multiple of kv_heads"),
    (dict(heads=2, kv_heads=4), 2, "multiple of kv_heads"),
    (dict(dtype=7), 4, "dtype"),
    (dict(head_dim=96), 5, "head_dim"),
    (dict(block_size=32, seq_len=1024), 5, "block_size"),
    (dict(top_k=18, block_size=64, seq_len=4096), 5, "top_k"),
    (dict(seq_len=1 << 27, block_size=1 << 20), 5, "seq_len"),
])
def test_forward_validation(kw, code, word):
    from sparse_long_context_moba_amd import _lib
    st = _lib.moba_forward(_p(**kw), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == code
    assert word in _lib.moba_last_error()
    st2, _ = _lib.moba_workspace_size(_p(**kw))
    assert st2 == code


def test_null_pointers_and_workspace():
    from sparse_long_context_moba_amd import _lib
    assert _lib.moba_forward(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None) == 1
    for i, name in enumerate(["q", "k", "v", "o", "block_idx"]):
        args = [FAKE] * 5
        args[i] = None
        st = _lib.moba_forward(_p(), *args, FAKE, 1 << 40, None)
        assert st == 1 and name in _lib.moba_last_error()
    st, need = _lib.moba_workspace_size(_p())
    assert st == 0 and need > 0
    assert _lib.moba_forward(_p(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == 6
    assert _lib.moba_forward(_p(), FAKE, FAKE, FAKE, FAKE, FAKE, None, need, None) == 6
    assert _lib.moba_forward(_p(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 8, need, None) == 6
    assert _lib.moba_dense_forward(_p(seq_len=1000, block_size=1000, head_dim=96), FAKE, FAKE, FAKE, FAKE, None) == 5
    assert _lib.moba_dense_forward(_p(), None, FAKE, FAKE, FAKE, None) == 1
    assert _lib.moba_debug_pool(_p(), FAKE, None, FAKE, need, None) == 1
    assert _lib.moba_debug_gate_topk(_p(), FAKE, FAKE, None, FAKE, need, None) == 1


def test_topk_beyond_blocks_is_clamped_not_an_error():
    from sparse_long_context_moba_amd import _lib
    st, a = _lib.moba_workspace_size(_p(top_k=4, seq_len=1024, block_size=256))
    st2, b = _lib.moba_workspace_size(_p(top_k=400, seq_len=1024, block_size=256))
    assert st == 0 and st2 == 0 and a == b


def test_workspace_of_named_workloads_fits_hbm():
    import synth
    from sparse_long_context_moba_amd import _lib
    for name in synth.WORKLOAD_ORDER:
        w = synth.WORKLOADS[name]
        p = _p(batch=w.batch, heads=w.heads, seq_len=w.seq_len, head_dim=w.head_dim,
               block_size=w.block_size, top_k=w.top_k, causal=int(w.causal),
               dtype=1 if w.dtype == "bf16" else 0)
        st, n = _lib.moba_workspace_size(p)
        assert st == 0, _lib.moba_last_error()
        assert 0 < n < 64 << 30, (name, n)


def test_short_last_block_is_accepted():
    """seq_len need not be a multiple of block_size (the last block is
    short); the kernels only need multiples of 64."""
    from sparse_long_context_moba_amd import _lib
    st, n = _lib.moba_workspace_size(_p(seq_len=1216, block_size=256))
    assert st == 0 and n > 0, _lib.moba_last_error()


def test_varlen_validation_and_workspace():
    from sparse_long_context_moba_amd import _lib
    cu = [0, 576, 1600, 1792]
    p = _p(batch=3, seq_len=1792, block_size=128)
    st, need = _lib.moba_workspace_size_varlen(p, cu)
    assert st == 0, _lib.moba_last_error()
    # one launch chain for the whole batch: its workspace holds every
    # sequence's lists and partials at once (more than the largest alone)
    per = [_lib.moba_workspace_size(_p(batch=1, seq_len=b - a, block_size=128))[1] for a, b in zip(cu, cu[1:])]
    assert need > max(per)
    # a one-sequence varlen batch needs the single problem's workspace plus its table
    st1, one = _lib.moba_workspace_size_varlen(_p(batch=1, seq_len=1000, block_size=128), [0, 1000])
    assert st1 == 0 and one >= _lib.moba_workspace_size(_p(batch=1, seq_len=1000, block_size=128))[1]
    big = 1 << 27
    cases = [
        (dict(cu=None), 1, "cu_seqlens"),
        (dict(cu=[1, 576, 1600, 1792]), 3, "cu_seqlens[0]"),
        (dict(p=_p(batch=2, seq_len=1792, block_size=128)), 3, "batch"),
        (dict(p=_p(batch=3, seq_len=1700, block_size=128)), 3, "seq_len"),
        (dict(cu=[0, 600, 600 + big, 700 + big], p=_p(batch=3, seq_len=700 + big, block_size=128)), 5, "2^27"),
        (dict(cu=[0, 576, 576, 1792]), 2, "sequence 1"),
    ]
    for kw, code, word in cases:
        c = kw.get("cu", cu)
        pp = kw.get("p", p)
        st, _ = _lib.moba_workspace_size_varlen(pp, c, None if c is not None else 3)
        assert st == code, (kw, _lib.moba_last_error())
        assert word in _lib.moba_last_error(), (kw, _lib.moba_last_error())
        st = _lib.moba_forward_varlen(pp, c, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None,
                                      n_seqs=None if c is not None else 3)
        assert st == code
    # too small a workspace is rejected before any launch
    assert _lib.moba_forward_varlen(p, cu, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == 6
    assert _lib.moba_forward_varlen(p, cu, None, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == 1


def test_any_sequence_length_is_accepted():
    """Lengths need not be multiples of 64 (a partial last tile of queries
    and keys is masked), for the forward and the backward; block_size
    still must be."""
    from sparse_long_context_moba_amd import _lib
    for S, Bs in ((1000, 128), (77, 64), (1, 64), (2049, 512), (33023, 512)):
        st, n = _lib.moba_workspace_size(_p(seq_len=S, block_size=Bs))
        assert st == 0 and n > 0, (S, Bs, _lib.moba_last_error())
    for S, Bs in ((1000, 128), (77, 64), (1, 64)):
        st, n = _lib.moba_backward_workspace_size(_p(seq_len=S, block_size=Bs))
        assert st == 0 and n > 0, (S, Bs, _lib.moba_last_error())
    st, _ = _lib.moba_workspace_size_varlen(_p(batch=3, seq_len=3126, block_size=64), [0, 1000, 1077, 3126])
    assert st == 0, _lib.moba_last_error()


def test_struct_layout_matches_header():
    """moba_problem_t: six int64, four int32, one int64, two int32 = 80 bytes,
    kv_heads at byte 64."""
    from sparse_long_context_moba_amd._lib import moba_problem_t
    assert ctypes.sizeof(moba_problem_t) == 80
    assert moba_problem_t.kv_heads.offset == 64
    assert moba_problem_t.gate_shared.offset == 72


def test_grouped_query_heads_workspace():
    """Key/value heads shrink the pooled-key arrays only: per-query-head
    buffers (counts, ranks, lists, partials) keep their size, and a shared
    gate needs no extra workspace."""
    from sparse_long_context_moba_amd import _lib
    st, mha = _lib.moba_workspace_size(_p(heads=8))
    st2, gqa = _lib.moba_workspace_size(_p(heads=8, kv_heads=2))
    st3, sh = _lib.moba_workspace_size(_p(heads=8, kv_heads=2, gate_shared=1))
    st4, same = _lib.moba_workspace_size(_p(heads=8, kv_heads=8))
    assert st == st2 == st3 == st4 == 0, _lib.moba_last_error()
    assert gqa < mha and sh == gqa and same == mha
    # pooled keys: fp64 + fp32 + bf16 hi/lo per coordinate, and an fp32 norm, per (kv head, block)
    nb, D = 1024 // 256, 128
    up = lambda x: (x + 255) // 256 * 256
    saved = sum(up(8 * nb * D * e) - up(2 * nb * D * e) for e in (8, 4, 2, 2)) + up(8 * nb * 4) - up(2 * nb * 4)
    assert mha - gqa == saved


def test_varlen_backward_validation():
    """moba_backward_varlen plans every sequence as its own uniform backward
    (bf16, any length) before anything is launched: an error names the
    sequence; the workspace is the largest sequence's."""
    from sparse_long_context_moba_amd import _lib
    cu = [0, 576, 1600, 1792]
    p = _p(batch=3, seq_len=1792, block_size=128)
    st, need = _lib.moba_backward_workspace_size_varlen(p, cu)
    assert st == 0, _lib.moba_last_error()
    per = [_lib.moba_backward_workspace_size(_p(batch=1, seq_len=b - a, block_size=128))[1]
           for a, b in zip(cu, cu[1:])]
    assert need == max(per)
    # ragged lengths are accepted; a sequence beyond the backward's block
    # limit (16384 blocks) is named
    st, _ = _lib.moba_backward_workspace_size_varlen(_p(batch=3, seq_len=1790, block_size=128), [0, 576, 1598, 1790])
    assert st == 0, _lib.moba_last_error()
    big = [0, 576, 576 + 64 * 16385]
    st, _ = _lib.moba_backward_workspace_size_varlen(_p(batch=2, seq_len=big[-1], block_size=64), big)
    assert st == 5 and "sequence 1" in _lib.moba_last_error()
    # fp32 inputs, batch and seq_len disagreeing with cu_seqlens
    assert _lib.moba_backward_workspace_size_varlen(_p(batch=3, seq_len=1792, block_size=128, dtype=0), cu)[0] == 5
    assert _lib.moba_backward_workspace_size_varlen(_p(batch=2, seq_len=1792, block_size=128), cu)[0] == 3
    args = [FAKE] * 10
    assert _lib.moba_backward_varlen(p, cu, *args, FAKE, need - 1, None) == 6
    for i, name in enumerate(["q", "k", "v", "o", "dout", "block_idx", "lse", "dq", "dk", "dv"]):
        a2 = list(args)
        a2[i] = None
        assert _lib.moba_backward_varlen(p, cu, *a2, FAKE, need, None) == 1 and name in _lib.moba_last_error()
    # the forward with log-sum-exp checks lse like the other outputs
    st, fneed = _lib.moba_workspace_size_varlen(p, cu)
    assert st == 0
    assert _lib.moba_forward_varlen_lse(p, cu, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, fneed, None) == 1
    assert "lse" in _lib.moba_last_error()


def test_backward_and_lse_validation():
    """moba_forward_lse and moba_backward validate on the host like
    moba_forward: bf16 only for the backward, every pointer named, the
    workspace size checked before anything is launched."""
    from sparse_long_context_moba_amd import _lib
    st, need = _lib.moba_backward_workspace_size(_p())
    st_f, fwd = _lib.moba_workspace_size(_p())
    assert st == 0 and st_f == 0 and need > fwd, _lib.moba_last_error()
    st, _ = _lib.moba_backward_workspace_size(_p(dtype=0))
    assert st == 5 and "bf16" in _lib.moba_last_error()
    st, _ = _lib.moba_backward_workspace_size(_p(top_k=0))
    assert st == 3
    names = ["q", "k", "v", "o", "dout", "block_idx", "lse", "dq", "dk", "dv"]
    for i, name in enumerate(names):
        args = [FAKE] * 10
        args[i] = None
        st = _lib.moba_backward(_p(), *args, FAKE, need, None)
        assert st == 1 and name in _lib.moba_last_error(), (name, _lib.moba_last_error())
    assert _lib.moba_backward(_p(), *([FAKE] * 10), FAKE, need - 1, None) == 6
    assert _lib.moba_backward(_p(), *([FAKE] * 10), FAKE + 8, need, None) == 6
    assert _lib.moba_backward(_p(dtype=0), *([FAKE] * 10), FAKE, need, None) == 5
    # the forward with the log-sum-exp: same workspace as the forward, lse required
    assert _lib.moba_forward_lse(_p(), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, fwd, None) == 1
    assert "lse" in _lib.moba_last_error()
    assert _lib.moba_forward_lse(_p(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, fwd - 1, None) == 6
    assert _lib.moba_forward_lse(_p(top_k=0), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, fwd, None) == 3


def test_python_buffer_checks_reject_wrong_buffers():
    """forward() and backward() check caller-supplied buffers before any
    call: a wrong shape, dtype, device or layout raises ValueError naming the
    buffer (checked here with CPU tensors standing for the device)."""
    import torch
    import sparse_long_context_moba_amd as moba
    q = torch.zeros(1, 2, 128, 64, dtype=torch.bfloat16)
    cpu = torch.device("cpu")
    ok = torch.zeros(1, 2, 128, 64, dtype=torch.bfloat16)
    assert moba.check_buffer(ok, "out", q.shape, q.dtype, cpu) is ok
    bad = [
        (torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16), "shape"),
        (torch.zeros(1, 2, 128, 64, dtype=torch.float32), "bfloat16"),
        (torch.zeros(1, 2, 64, 128, dtype=torch.bfloat16).transpose(2, 3), "contiguous"),
        (torch.zeros(1, 2, 128, 64, dtype=torch.bfloat16, device="meta"), "cpu"),
        (None, "tensor"),
    ]
    for t, word in bad:
        with pytest.raises(ValueError, match=word):
            moba.check_buffer(t, "out", q.shape, q.dtype, cpu)
    idx_shape = (1, 2, 128, 3)
    with pytest.raises(ValueError, match="idx"):
        moba.check_buffer(torch.zeros(idx_shape, dtype=torch.int64), "idx", idx_shape, torch.int32, cpu)
    with pytest.raises(ValueError, match="idx"):
        moba.check_buffer(torch.zeros((1, 2, 128, 2), dtype=torch.int32), "idx", idx_shape, torch.int32, cpu)
    with pytest.raises(ValueError, match="lse"):
        moba.check_buffer(torch.zeros((1, 2, 127), dtype=torch.float32), "lse", (1, 2, 128), torch.float32, cpu)
    ws = torch.zeros(100, dtype=torch.float32)
    assert moba.check_workspace(ws, 400, cpu) == 400
    with pytest.raises(ValueError, match="needs 401"):
        moba.check_workspace(ws, 401, cpu)
    with pytest.raises(ValueError, match="contiguous"):
        moba.check_workspace(torch.zeros(200, dtype=torch.uint8)[::2], 10, cpu)
