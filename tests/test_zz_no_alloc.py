"""convrot_linear_noalloc (the layer for callers that cannot allocate device
memory) against convrot_linear, byte for byte, through the C ABI.

Two calls in a row on one GPU, the second with a smaller input, so the
second reuses the library's scratch array after a larger call left its bytes
there; then layers whose slice of codes does not fit the array in one piece
(K = 12288: 2720 tokens per slice), so the call runs in several slices.  Each
result must equal convrot_linear's with its own workspace (same kernels, same
slices where both slice, and slicing never changes the bytes).
"""
import ctypes

import numpy as np
import pytest
import torch

from tests._util import to_dev_bf16
from w8a8_rotated_int8_convrot_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from w8a8_rotated_int8_convrot_amd import binding
    binding.lib()
    return binding


def layer(B, M, K, N, seed, bias=True):
    r = np.random.default_rng(seed)
    x = r.standard_t(4, (M, K))
    x[:, r.choice(K, 4, replace=False)] *= 20.0
    xb = to_dev_bf16(synth.to_bf16_bits(x), DEV)
    w = torch.from_numpy((r.standard_normal((N, K)) * 0.02).astype(np.float32)).to(DEV)
    wq, s_w = B.convrot_prepare_weight(w, 128)
    b = to_dev_bf16(synth.to_bf16_bits(r.standard_normal(N) * 0.01), DEV) if bias else None
    return xb, wq, s_w, b


def noalloc_abi(B, x, wq, s_w, bias, y, g=128):
    """The entry point called directly through ctypes (no binding logic)."""
    M, K = x.shape
    N = wq.shape[0]
    rc = B.lib().convrot_linear_noalloc(x.data_ptr(), M, K, wq.data_ptr(), s_w.data_ptr(), N, g,
                                        None if bias is None else bias.data_ptr(), y.data_ptr(),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, B.last_error()


def same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_two_calls_in_a_row_second_smaller(B):
    x1, wq1, s1, b1 = layer(B, 3000, 3072, 4096, 1)
    x2, wq2, s2, b2 = layer(B, 333, 1024, 1000, 2, bias=False)
    y1 = torch.empty((3000, 4096), dtype=torch.bfloat16, device=DEV)
    y2 = torch.empty((333, 1000), dtype=torch.bfloat16, device=DEV)
    noalloc_abi(B, x1, wq1, s1, b1, y1)
    noalloc_abi(B, x2, wq2, s2, b2, y2)
    torch.cuda.synchronize()
    assert same(y1, B.convrot_linear(x1, wq1, s1, 128, b1))
    assert same(y2, B.convrot_linear(x2, wq2, s2, 128, b2))


def test_sliced_through_the_scratch_array(B):
    # K = 12288: 32 MiB holds 2720 tokens' codes and scales, so 4608 tokens
    # run in two slices; then a smaller sliced call right after
    for M, K, N, seed in ((4608, 12288, 3072, 3), (3000, 12288, 1536, 4)):
        x, wq, s_w, b = layer(B, M, K, N, seed)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        noalloc_abi(B, x, wq, s_w, b, y)
        torch.cuda.synchronize()
        assert same(y, B.convrot_linear(x, wq, s_w, 128, b)), (M, K, N)


def test_binding_and_empty_batch(B):
    x, wq, s_w, b = layer(B, 64, 512, 300, 5)
    assert same(B.convrot_linear_noalloc(x, wq, s_w, 128, b), B.convrot_linear(x, wq, s_w, 128, b))
    y0 = B.convrot_linear_noalloc(x[:0], wq, s_w, 128, b)
    assert y0.shape == (0, 300)
