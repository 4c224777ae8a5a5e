"""moba_forward_noalloc, the allocation-free forward, through the C ABI:
two calls in a row (the second on a smaller problem, so the scratch array
holds the first call's leftovers) must give exactly moba_forward's outputs
with a caller-allocated workspace, and a problem above the scratch size
must be rejected before anything runs."""
import numpy as np
import pytest
import torch

from tests.parity import say

pytestmark = pytest.mark.gpu


def _problem(B, H, S, D, Bs, top_k, causal, dtype):
    from sparse_long_context_moba_amd import _lib
    return _lib.moba_problem_t(B, H, S, D, Bs, top_k, 1 if causal else 0, 1 if dtype == torch.bfloat16 else 0,
                               0, 0, 0, 0, 0)


def _inputs(seed, B, H, S, D, Bs, dtype):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, S, D, generator=g)
    k = torch.randn(B, H, S, D, generator=g)
    nb = -(-S // Bs)
    k += (0.5 * torch.randn(B, H, nb, 1, D, generator=g)).expand(B, H, nb, Bs, D).reshape(B, H, nb * Bs, D)[:, :, :S]
    v = torch.randn(B, H, S, D, generator=g)
    return [x.to(dtype).cuda().contiguous() for x in (q, k, v)]


def _both(shape, seed):
    """Outputs of moba_forward (torch workspace) and moba_forward_noalloc."""
    from sparse_long_context_moba_amd import _lib
    B, H, S, D, Bs, top_k, causal, dtype = shape
    q, k, v = _inputs(seed, B, H, S, D, Bs, dtype)
    p = _problem(*shape)
    st, need = _lib.moba_workspace_size(p)
    assert st == 0 and need <= _lib.NOALLOC_SCRATCH_BYTES
    stream = torch.cuda.current_stream().cuda_stream
    o_ref, o_na = torch.empty_like(q), torch.full_like(q, 3.0)
    i_ref = torch.empty((B, H, S, top_k), dtype=torch.int32, device="cuda")
    i_na = torch.full_like(i_ref, -7)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    assert _lib.moba_forward(p, q.data_ptr(), k.data_ptr(), v.data_ptr(), o_ref.data_ptr(), i_ref.data_ptr(),
                             ws.data_ptr(), need, stream) == 0, _lib.moba_last_error()
    st = _lib.moba_forward_noalloc(p, q.data_ptr(), k.data_ptr(), v.data_ptr(), o_na.data_ptr(), i_na.data_ptr(),
                                   stream)
    assert st == 0, _lib.moba_last_error()
    torch.cuda.synchronize()
    return o_ref, i_ref, o_na, i_na


def test_noalloc_matches_forward_on_two_calls_in_a_row():
    first = (1, 4, 4096, 128, 256, 3, True, torch.bfloat16)
    second = (1, 2, 1024, 64, 128, 2, True, torch.bfloat16)  # smaller: stale scratch from the first call
    for i, (shape, seed) in enumerate(((first, 1), (second, 2))):
        say(f"[gpu] noalloc call {i + 1}: {shape}")
        o_ref, i_ref, o_na, i_na = _both(shape, seed)
        assert torch.equal(i_na, i_ref), f"call {i + 1}: block indices differ"
        assert torch.equal(o_na.view(torch.int16), o_ref.view(torch.int16)), f"call {i + 1}: outputs differ"
    say("[gpu] noalloc: both calls bit-identical to moba_forward")


def test_noalloc_fp32_noncausal_after_bf16():
    shape = (1, 2, 2048, 64, 256, 3, False, torch.float32)
    say(f"[gpu] noalloc fp32: {shape}")
    o_ref, i_ref, o_na, i_na = _both(shape, 3)
    assert torch.equal(i_na, i_ref)
    assert torch.equal(o_na.view(torch.int32), o_ref.view(torch.int32))


def test_noalloc_rejects_problems_above_the_scratch_size():
    from sparse_long_context_moba_amd import _lib
    q, k, v = _inputs(4, 1, 1, 256, 64, 64, torch.bfloat16)
    o = torch.full_like(q, 5.0)
    idx = torch.full((1, 1, 256, 3), 9, dtype=torch.int32, device="cuda")
    big = _problem(1, 32, 32768, 128, 512, 3, True, torch.bfloat16)  # needs about 540 MiB
    st = _lib.moba_forward_noalloc(big, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), idx.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
    assert st == 6 and "moba_forward_noalloc" in _lib.moba_last_error()
    torch.cuda.synchronize()
    assert bool((o == 5.0).all()) and bool((idx == 9).all())
