"""kda_prefill_noalloc, the entry point for callers that cannot allocate
(graph capture, tight serving loops): called through the C ABI, its core rows
and carried state are bitwise those of kda_prefill on the same inputs, on two
calls in a row (the second on a smaller input, so the library's scratch array
still holds the first call's blocks), and at a size that takes several
segments of the array."""
import ctypes

import numpy as np
import pytest
import torch

import gated_delta_rule_bounded_amd as kda
from kda_cases import core_case, cuda, gpu_prefill, pad_rows, say

pytestmark = pytest.mark.gpu


def _noalloc_c_abi(case, T, T_pad, C, scale, fill=0.0):
    """The entry point called through ctypes with raw device pointers."""
    H, D = case["q"].shape[1:]
    ins = [cuda(pad_rows(case[n][:T], T_pad, fill)) for n in ("q", "k", "v", "gate", "beta")]
    st = cuda(case["S0"]).contiguous()
    core = torch.full((T_pad, H, D), 7.0, dtype=torch.float32, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = kda._lib.lib.kda_prefill_noalloc(*[p(t) for t in ins], p(st), p(core), T, T_pad, H, D, C,
                                          ctypes.c_float(scale), stream)
    assert rc == 0, kda.last_error()
    torch.cuda.synchronize()
    return core.cpu().numpy(), st.cpu().numpy()


@pytest.mark.parametrize("first,second", [
    # (T, T_pad, H, D, C), the second call smaller than the first
    ((300, 320, 4, 128, 64), (57, 64, 2, 16, 16)),
    # the prefill workload's shape: 4096 tokens x 32 heads do not fit the
    # 64 MiB array in one segment (4.6 MiB of blocks per chunk), so the call
    # walks several segments; then a ragged, smaller one
    ((4096, 4096, 32, 128, 64), (1000, 1024, 32, 128, 64)),
])
def test_noalloc_equals_kda_prefill_twice(first, second):
    for n, (T, T_pad, H, D, C) in enumerate((first, second)):
        case = core_case(T, H, D, 1900 + 17 * n + T, 0.05, qkv_bf16=True)
        scale = D ** -0.5
        say("prefill_noalloc", n, T, T_pad, H, D, C)
        core_a, S_a = _noalloc_c_abi(case, T, T_pad, C, scale, fill=np.nan)
        core_b, S_b = gpu_prefill(case, T, T_pad, C, scale, fill=np.nan)
        np.testing.assert_array_equal(core_a[:T], core_b[:T], err_msg=f"call {n} core")
        np.testing.assert_array_equal(S_a, S_b, err_msg=f"call {n} state")
        assert np.all(core_a[T:] == 7.0), f"call {n}: core rows past T written"


def test_noalloc_rejects_heads_beyond_the_array():
    # one chunk of 500 heads x 128 at chunk 64 needs ~72 MiB of blocks: more
    # than the 64 MiB array, refused before any launch
    H, D, C, T = 500, 128, 64, 64
    x = torch.zeros(T, H, D, device="cuda")
    b = torch.zeros(T, H, device="cuda")
    st = torch.zeros(H, D, D, device="cuda")
    with pytest.raises(kda.KdaError, match="scratch"):
        kda.kda_prefill_noalloc(x, x.clone(), x.clone(), x.clone(), b, st,
                                torch.zeros(T, H, D, device="cuda"), T=T, T_pad=T, heads=H,
                                head_dim=D, chunk=C, scale=0.1)
