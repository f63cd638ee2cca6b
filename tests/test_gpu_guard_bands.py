"""Stores stay inside their buffers: every output of the C ABI is placed inside
a larger device buffer whose bytes before and after it hold a fixed pattern,
the call runs on ragged shapes (M, N not multiples of any tile; every GEMM
tile forced in turn; both rotate+quant kernels; the half-height tail split),
and the pattern must be intact afterwards.  The outputs themselves must equal
those of the same call into ordinary tensors.  Nothing here writes out of
bounds on purpose: a store past an output would land in the band and fail
the test, not fault.
"""
import ctypes

import numpy as np
import pytest
import torch

from tests._util import to_dev_bf16
from w8a8_rotated_int8_convrot_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BAND = 4096          # guard bytes on each side
PATTERN = 0xA5


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from w8a8_rotated_int8_convrot_amd import binding
    binding.lib()
    return binding


class Banded:
    """A device buffer of `nbytes` with BAND pattern bytes on each side."""

    def __init__(self, nbytes):
        self.n = nbytes
        self.buf = torch.full((BAND + nbytes + BAND,), PATTERN, dtype=torch.uint8, device=DEV)

    def view(self, dtype, shape):
        t = self.buf[BAND:BAND + self.n].view(dtype)
        return t.view(*shape)

    def ptr(self):
        return self.buf.data_ptr() + BAND

    def intact(self):
        torch.cuda.synchronize()
        head = self.buf[:BAND].cpu().numpy()
        tail = self.buf[BAND + self.n:].cpu().numpy()
        return bool(np.all(head == PATTERN) and np.all(tail == PATTERN))


def rand_i8(shape, seed):
    return np.random.default_rng(seed).integers(-127, 128, size=shape, dtype=np.int64).astype(np.int8)


def stream():
    return torch.cuda.current_stream().cuda_stream


def gemm_case(B, M, N, K, seed):
    a = torch.from_numpy(rand_i8((M, K), seed)).to(DEV)
    b = torch.from_numpy(rand_i8((N, K), seed + 1)).to(DEV)
    r = np.random.default_rng(seed)
    s_x = torch.from_numpy((r.random(M) * 0.2 + 1e-3).astype(np.float32)).to(DEV)
    s_w = torch.tensor([1.3e-4], dtype=torch.float32, device=DEV)
    bias = to_dev_bf16(synth.to_bf16_bits(r.standard_normal(N) * 0.01), DEV)
    # int32 products
    acc = Banded(M * N * 4)
    rc = B.lib().convrot_gemm_i32(a.data_ptr(), b.data_ptr(), M, N, K, ctypes.c_void_p(acc.ptr()), stream())
    assert rc == 0, B.last_error()
    assert acc.intact(), "int32 store outside acc"
    assert torch.equal(acc.view(torch.int32, (M, N)), B.convrot_gemm_i32(a, b))
    # dequant + bias epilogue
    y = Banded(M * N * 2)
    B.convrot_gemm_dequant(a, s_x, b, s_w, bias, out=y.view(torch.bfloat16, (M, N)))
    assert y.intact(), "bf16 store outside y"
    ref = B.convrot_gemm_dequant(a, s_x, b, s_w, bias)
    assert torch.equal(y.view(torch.int16, (M, N)), ref.view(torch.int16))


@pytest.mark.parametrize("tile", ["big", "big8", "wide", "wide128", "mid", "skinny", "skinny16", "half", "p128", "phalf", "tall", "ptall",
                                  "m32", "m64", "m128"])
@pytest.mark.parametrize("M,N,K", [(301, 1001, 384), (17, 35, 256), (1111, 777, 128)])
def test_gemm_stores_stay_inside_on_every_tile(B, tile, M, N, K, monkeypatch):
    monkeypatch.setenv("CONVROT_GEMM_TILE", tile)
    gemm_case(B, M, N, K, M + N + K)


@pytest.mark.parametrize("tile", ["p128", "ptall"])
@pytest.mark.parametrize("M,N,K", [(2500, 9001, 384), (4700, 12290, 640)])
def test_gemm_stores_stay_inside_persistent_tiles(B, tile, M, N, K, monkeypatch):
    # more tiles than CUs: each persistent workgroup runs several, ragged in
    # both M and N
    monkeypatch.setenv("CONVROT_GEMM_TILE", tile)
    gemm_case(B, M, N, K, 11 * M + N)


@pytest.mark.parametrize("tile", ["ksplit"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (13, 1001, 384), (16, 3001, 4096)])
def test_gemm_stores_stay_inside_ksplit_tiles(B, tile, M, N, K, monkeypatch):
    monkeypatch.setenv("CONVROT_GEMM_TILE", tile)
    gemm_case(B, M, N, K, 13 * M + N)


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (15, 12287, 512), (129, 3001, 384), (2001, 12283, 384)])
def test_gemm_stores_stay_inside_automatic_tiles(B, M, N, K):
    # 2001 x 12283: ragged 192 x 288 tiles, some workgroups running two (the
    # 384 x 192 tiles with their half-height tail are covered by the forced
    # persistent tile "p128" above)
    gemm_case(B, M, N, K, 7 * M + N)


@pytest.mark.parametrize("M,K,g", [(3, 384, 128), (301, 3072, 128), (77, 1024, 256),       # row kernel
                                   (701, 3072, 128), (33, 12288, 128), (129, 16384, 256),   # block kernel
                                   (3, 33024, 256)])                                        # two-pass rows
def test_rotate_quant_stores_stay_inside(B, M, K, g):
    r = np.random.default_rng(M + K)
    x = to_dev_bf16(synth.to_bf16_bits(r.standard_normal((M, K))), DEV)
    q = Banded(M * K)
    s = Banded(M * 4)
    B.convrot_rotate_quant(x, g, q.view(torch.int8, (M, K)), s.view(torch.float32, (M,)))
    assert q.intact() and s.intact()
    q_ref, s_ref = B.convrot_rotate_quant(x, g)
    assert torch.equal(q.view(torch.int8, (M, K)), q_ref)
    assert torch.equal(s.view(torch.float32, (M,)), s_ref)


@pytest.mark.parametrize("M,K,N", [(301, 384, 1001), (1000, 256, 96), (33, 12288, 3001)])
def test_linear_stays_inside_output_and_workspace(B, M, K, N):
    # (1000, 256, 96): M > 2N, so the call runs in slices through the workspace
    r = np.random.default_rng(M * N)
    x = to_dev_bf16(synth.to_bf16_bits(r.standard_t(4, (M, K))), DEV)
    w = torch.from_numpy((r.standard_normal((N, K)) * 0.02).astype(np.float32)).to(DEV)
    wq, s_w = B.convrot_prepare_weight(w, 128)
    bias = to_dev_bf16(synth.to_bf16_bits(r.standard_normal(N) * 0.01), DEV)
    nws = B.convrot_linear_workspace(M, K, N)
    ws = Banded(nws)
    y = Banded(M * N * 2)
    B.convrot_linear(x, wq, s_w, 128, bias, out=y.view(torch.bfloat16, (M, N)),
                     workspace=ws.view(torch.uint8, (nws,)))
    assert y.intact(), "output store outside y"
    assert ws.intact(), "workspace store outside the workspace"
    ref = B.convrot_linear(x, wq, s_w, 128, bias)
    assert torch.equal(y.view(torch.int16, (M, N)), ref.view(torch.int16))


def test_prepare_weight_stays_inside(B):
    N, K = 333, 1152
    w = torch.from_numpy((np.random.default_rng(5).standard_normal((N, K)) * 0.02).astype(np.float32)).to(DEV)
    wq = Banded(N * K)
    sc = Banded(4)
    nws = B.convrot_prepare_weight_workspace(N, K)
    ws = Banded(nws)
    rc = B.lib().convrot_prepare_weight(w.data_ptr(), B.CONVROT_F32, N, K, 128, ctypes.c_void_p(wq.ptr()),
                                        ctypes.c_void_p(sc.ptr()), ctypes.c_void_p(ws.ptr()), nws, stream())
    assert rc == 0, B.last_error()
    assert wq.intact() and sc.intact() and ws.intact()
    wq_ref, s_ref = B.convrot_prepare_weight(w, 128)
    assert torch.equal(wq.view(torch.int8, (N, K)), wq_ref)
    assert torch.equal(sc.view(torch.float32, (1,)), s_ref)
