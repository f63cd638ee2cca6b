"""GPU parity of the layer's variants against the oracle: fp16 in place of
bf16 for the activation, the bias and the output (page "int8 Compute", "What
stays on the default path": compute is offered in BF16 or FP16), and one weight
scale per output channel (page "Explanation of INT8 ConvRot", format table:
row-wise scaling).  Integer work (codes, scales) is compared bit for bit, and
so are the outputs: both sides round the same fp32 value once to fp16 / bf16.
"""
import numpy as np
import pytest
import torch

import oracle
from w8a8_rotated_int8_convrot_amd import binding as B
from w8a8_rotated_int8_convrot_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def f16_bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def dev16(bits: np.ndarray, io: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)
    return t.view(torch.float16 if io == "f16" else torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def act(M, K, seed, io):
    r = np.random.default_rng(seed)
    x = r.standard_t(4, (M, K))
    x[:, r.choice(K, 3, replace=False)] *= 25.0
    x[0] = 0.0                                              # a zero token
    return f16_bits(x) if io == "f16" else synth.to_bf16_bits(x)


# the row kernel (M*K <= 2^21, K < 8192) and the block kernel
@pytest.mark.parametrize("M,K,g", [(37, 3072, 128), (701, 3072, 128), (523, 4096, 256), (9, 16384, 256)])
def test_rotate_quant_f16_bit_exact(M, K, g):
    x = act(M, K, M + K, "f16")
    q, s = B.convrot_rotate_quant_ex(dev16(x, "f16"), g)
    q_ref, s_ref = oracle.quant_act(x, g, io="f16")
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy(), s_ref)


@pytest.mark.parametrize("wdt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("mode", ["row", "tensor"])
@pytest.mark.parametrize("N,K,g", [(300, 3072, 128), (2100, 1024, 256)])
def test_prepare_weight_variants_bit_exact(wdt, mode, N, K, g):
    r = np.random.default_rng(N + K)
    w = (r.standard_normal((N, K)) * 0.02 * r.uniform(0.1, 4.0, (N, 1))).astype(np.float32)
    w[3] = 0.0                                              # a zero channel
    if wdt == "f32":
        wd, w_exact = torch.from_numpy(w).to(DEV), w
    elif wdt == "bf16":
        bits = synth.to_bf16_bits(w)
        wd, w_exact = dev16(bits, "bf16"), oracle.bf16_bits_to_f32(bits)
    else:
        bits = f16_bits(w)
        wd, w_exact = dev16(bits, "f16"), bits.view(np.float16).astype(np.float32)
    wq, s = B.convrot_prepare_weight_ex(wd, g, mode)
    if mode == "row":
        wq_ref, s_ref = oracle.quant_weight_rows(w_exact, g)
    else:
        wq_ref, s1 = oracle.quant_weight(w_exact, g)
        s_ref = np.array([s1], dtype=np.float32)
    assert np.array_equal(wq.cpu().numpy(), wq_ref)
    assert np.array_equal(s.cpu().numpy(), s_ref)


@pytest.mark.parametrize("io", ["bf16", "f16"])
@pytest.mark.parametrize("mode", ["row", "tensor"])
@pytest.mark.parametrize("M,N,K", [(300, 1001, 384), (1111, 777, 640), (16, 3000, 1024)])
def test_gemm_dequant_variants_bit_exact(io, mode, M, N, K):
    r = np.random.default_rng(M * 3 + N + K)
    a = r.integers(-127, 128, (M, K), dtype=np.int8)
    b = r.integers(-127, 128, (N, K), dtype=np.int8)
    s_x = (r.random(M) * 0.2 + 1e-3).astype(np.float32)
    s_w = (r.random(N if mode == "row" else 1) * 2e-4 + 1e-6).astype(np.float32)
    bias = f16_bits(r.standard_normal(N) * 0.5) if io == "f16" else synth.to_bf16_bits(r.standard_normal(N) * 0.5)
    y = B.convrot_gemm_dequant_ex(torch.from_numpy(a).to(DEV), torch.from_numpy(s_x).to(DEV),
                                  torch.from_numpy(b).to(DEV), torch.from_numpy(s_w).to(DEV),
                                  dev16(bias, io),
                                  out_dtype=torch.float16 if io == "f16" else torch.bfloat16)
    acc = oracle.gemm_i32(a, b)
    ref = oracle.epilogue(acc, s_x, s_w if mode == "row" else s_w[0], bias, io=io)
    assert np.array_equal(host_bits(y), ref)


@pytest.mark.parametrize("io", ["bf16", "f16"])
@pytest.mark.parametrize("mode", ["row", "tensor"])
@pytest.mark.parametrize("M,K,N,g", [(257, 3072, 1000, 128), (1024, 4096, 640, 256)])
def test_linear_variants_end_to_end(io, mode, M, K, N, g):
    r = np.random.default_rng(M + K + N)
    x = act(M, K, M * 7 + K, io)
    w = (r.standard_normal((N, K)) * 0.02 * r.uniform(0.2, 3.0, (N, 1))).astype(np.float32)
    bias_f = r.standard_normal(N) * 0.01
    bias = f16_bits(bias_f) if io == "f16" else synth.to_bf16_bits(bias_f)
    wq, s_w = B.convrot_prepare_weight_ex(torch.from_numpy(w).to(DEV), g, mode)
    y = B.convrot_linear_ex(dev16(x, io), wq, s_w, g, dev16(bias, io))
    if mode == "row":
        wq_ref, s_ref = oracle.quant_weight_rows(w, g)
    else:
        wq_ref, s_ref = oracle.quant_weight(w, g)
    y_ref, _, _ = oracle.linear(x, wq_ref, s_ref, g, bias, io=io)
    assert np.array_equal(host_bits(y), y_ref)
    # and the variant layer approximates the unquantized product
    widen = (lambda b: b.view(np.float16).astype(np.float64)) if io == "f16" else \
        (lambda b: oracle.bf16_bits_to_f32(b).astype(np.float64))
    ref = widen(x) @ w.astype(np.float64).T + widen(bias)[None, :]
    assert oracle.nrmse(widen(y_ref), ref) < 0.05


@pytest.mark.parametrize("tile", ["big", "big8", "wide", "wide128", "mid", "skinny", "skinny16", "m32", "m64", "m128",
                                  "p128", "phalf", "tall", "ptall", "ksplit", "ksplit3072", "ksplit4096"])
def test_every_tile_runs_the_variant_epilogues(tile, monkeypatch):
    monkeypatch.setenv("CONVROT_GEMM_TILE", tile[:6] if tile.startswith("ksplit") else tile)
    r = np.random.default_rng(5)
    # the K-split tiles hold at most 16 tokens; at K = 3072 and 4096 the
    # K-split tile streams its operands through registers
    M, N, K = (13, 1001, int(tile[6:] or 384)) if tile.startswith("ksplit") else (300, 1001, 384)
    a = r.integers(-127, 128, (M, K), dtype=np.int8)
    b = r.integers(-127, 128, (N, K), dtype=np.int8)
    s_x = (r.random(M) * 0.2 + 1e-3).astype(np.float32)
    s_w = (r.random(N) * 2e-4 + 1e-6).astype(np.float32)
    bias = f16_bits(r.standard_normal(N) * 0.5)
    acc = oracle.gemm_i32(a, b)
    args = [torch.from_numpy(a).to(DEV), torch.from_numpy(s_x).to(DEV), torch.from_numpy(b).to(DEV)]
    y_row = B.convrot_gemm_dequant_ex(*args, torch.from_numpy(s_w).to(DEV), dev16(bias, "f16"),
                                      out_dtype=torch.float16)
    assert np.array_equal(host_bits(y_row), oracle.epilogue(acc, s_x, s_w, bias, io="f16"))
    y_t = B.convrot_gemm_dequant_ex(*args, torch.from_numpy(s_w[:1]).to(DEV), dev16(bias, "f16"),
                                    out_dtype=torch.float16)
    assert np.array_equal(host_bits(y_t), oracle.epilogue(acc, s_x, s_w[0], bias, io="f16"))
