"""gdn_prefill_chunked_noalloc: the prefill with its workspace in the
library's static device array, for callers that cannot allocate.  Called
through the C ABI and compared with gdn_prefill_chunked (a caller workspace)
on two calls in a row, the second smaller, and with the fp64 oracle; a call
beyond the array is refused before any HIP call and touches nothing."""
import ctypes

import numpy as np
import pytest

import gdn_inputs as gi
from gpu_helpers import assert_parity, dev, gpu_prefill, host, oracle_prefill, say

GDN_BF16, GDN_F32, GDN_ERROR_WORKSPACE = 1, 0, 3
SCRATCH_BYTES = 256 * 1024 * 1024


def _noalloc(x, o, S, *, scale):
    """gdn_prefill_chunked_noalloc through ctypes on the current stream."""
    import torch
    import gated_delta_rule_decode_amd as gdn
    bf = torch.bfloat16
    q, k, v, g, b = dev(x.q, bf), dev(x.k, bf), dev(x.v, bf), dev(x.g), dev(x.beta)
    cu = dev(x.cu_seqlens.astype(np.int32))
    s0 = dev(x.s0) if x.s0 is not None else None
    T, N = int(x.cu_seqlens[-1]), len(x.cu_seqlens) - 1
    st = gdn.lib().gdn_prefill_chunked_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), GDN_BF16, g.data_ptr(), b.data_ptr(),
        cu.data_ptr(), N, T, None if s0 is None else s0.data_ptr(), S.data_ptr(), o.data_ptr(),
        GDN_F32, x.H, x.HV, x.dk, x.dv, 64, ctypes.c_float(scale),
        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return st


def test_refused_beyond_the_array():
    """Host-only: a call whose workspace would exceed the array returns
    GDN_ERROR_WORKSPACE before anything is enqueued (no device is needed)."""
    import gated_delta_rule_decode_amd as gdn
    L = gdn.lib()
    assert gdn.prefill_workspace_bytes(1, 65536, 16, 32, 128, 128) > SCRATCH_BYTES
    fake = 0x10000
    st = L.gdn_prefill_chunked_noalloc(fake, fake, fake, GDN_BF16, fake, fake, fake, 1, 65536,
                                       None, fake, fake, GDN_F32, 16, 32, 128, 128, 64,
                                       ctypes.c_float(1.0), None)
    assert st == GDN_ERROR_WORKSPACE
    # argument errors keep their own status
    assert L.gdn_prefill_chunked_noalloc(fake, fake, fake, GDN_BF16, fake, fake, fake, 1, 100,
                                         None, fake, fake, GDN_F32, 16, 32, 96, 128, 64,
                                         ctypes.c_float(1.0), None) == 2
    assert L.gdn_prefill_chunked_noalloc(fake, fake, fake, GDN_BF16, fake, fake, fake, 0, 100,
                                         None, fake, fake, GDN_F32, 16, 32, 128, 128, 64,
                                         ctypes.c_float(1.0), None) == 0


@pytest.mark.gpu
def test_noalloc_equals_caller_workspace_twice(orc):
    """Two calls in a row, the second smaller (fewer tokens, heads and
    sequences): each equals gdn_prefill_chunked with a caller workspace bit
    for bit, and the oracle within the parity bars.  The array keeps the
    first call's contents when the second runs."""
    import torch
    import gated_delta_rule_decode_amd as gdn
    cases = [gi.make_prefill([2500, 1, 640, 1300], 4, 8, 128, 128, s0_std=0.02, seed=501),
             gi.make_prefill([300, 64], 2, 4, 128, 128, seed=502)]
    for i, x in enumerate(cases):
        T, N = int(x.cu_seqlens[-1]), len(x.cu_seqlens) - 1
        assert gdn.prefill_workspace_bytes(N, T, x.H, x.HV, 128, 128) <= SCRATCH_BYTES
        say(f"prefill no-alloc call {i}: lengths={list(x.lengths)} H={x.H} HV={x.HV}")
        o = torch.full((T, x.HV, 128), float("nan"), device="cuda")
        S = torch.full((N, x.HV, 128, 128), float("nan"), device="cuda")
        assert _noalloc(x, o, S, scale=128 ** -0.5) == 0
        o_ref_gpu, S_ref_gpu = gpu_prefill(x, scale=128 ** -0.5)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref_gpu) and torch.equal(S, S_ref_gpu), f"call {i}"
        o_ref, S_ref = oracle_prefill(orc, x, scale=128 ** -0.5)
        assert_parity(host(o), host(S), o_ref, S_ref, what=f"no-alloc call {i}",
                      cu=x.cu_seqlens)
