"""The default (dequantizing) path and the guarded layer on the GPU.

Page "int8 Compute" (InvokeAI docs), "When something goes wrong": a new
combination of layer shape and batch-size bucket is verified once against the
default path; on a disagreement or a kernel error a single warning is
written and the device stays on the default path for the rest of the run.

* The unpacked weight (dequantize, rotate back, round) is integer-and-rounding
  work done in a pinned fp32 order: bit-exact against the oracle.
* The default product accumulates in fp32 inside the matrix cores, in an
  order the oracle does not reproduce: every element is held to the bound
  |y - exact| <= ulp(exact) + K * 2^-24 * sum|x * w| (one output ulp, plus
  the worst case of an fp32 sum of K terms), and nearly every element must
  equal the oracle's rounding.
* The guard's decisions are driven from the host (a fault injected before
  the call): nothing here makes the GPU fail.
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
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def widen(bits: np.ndarray, io: str) -> np.ndarray:
    if io == "f16":
        return bits.view(np.float16).astype(np.float64)
    return oracle.bf16_bits_to_f32(bits).astype(np.float64)


def ulp(v: np.ndarray, io: str) -> np.ndarray:
    e = np.floor(np.log2(np.maximum(np.abs(v), 1e-300)))
    return 2.0 ** (np.maximum(e, -14) - 10) if io == "f16" else 2.0 ** (e - 7)


def weight(N, K, seed):
    r = np.random.default_rng(seed)
    w = (r.standard_normal((N, K)) * 0.02 * r.uniform(0.2, 3.0, (N, 1))).astype(np.float32)
    return w


def act(M, K, seed, io):
    r = np.random.default_rng(seed)
    x = r.standard_t(4, (M, K))
    x[:, r.choice(K, 3, replace=False)] *= 25.0
    return f16_bits(x) if io == "f16" else synth.to_bf16_bits(x)


def prepared(N, K, g, mode, seed):
    wq, s_w = B.convrot_prepare_weight_ex(torch.from_numpy(weight(N, K, seed)).to(DEV), g, scale_mode=mode)
    return wq, s_w


def assert_default_close(y_bits, x_bits, rows, wu_bits, bias_bits, io, K):
    y_ref, exact, mag = oracle.default_rows(x_bits, rows, wu_bits, bias_bits, io=io)
    got = widen(y_bits, io)
    bound = ulp(exact, io) + K * 2.0 ** -24 * mag + 1e-30
    bad = np.abs(got - exact) > bound
    assert not bad.any(), f"{bad.sum()} values outside the bound, first at {np.argwhere(bad)[:3]}"
    same = (y_bits == y_ref) | ((got == 0) & (widen(y_ref, io) == 0))
    assert same.mean() >= 0.99, same.mean()
    assert oracle.nrmse(got, widen(y_ref, io)) <= 1e-3


# ---------------------------------------------------------------- default path

@pytest.mark.parametrize("io", ["bf16", "f16"])
@pytest.mark.parametrize("mode", ["tensor", "row"])
@pytest.mark.parametrize("N,K,g", [(300, 3072, 128), (77, 12288, 256), (2048, 1024, 128), (5, 16384, 256)])
def test_unpack_weight_bit_exact(io, mode, N, K, g):
    wq, s_w = prepared(N, K, g, mode, N + K)
    wu = B.convrot_unpack_weight(wq, s_w, g, out_dtype=torch.float16 if io == "f16" else torch.bfloat16)
    ref = oracle.unpack_weight(wq.cpu().numpy(), s_w.cpu().numpy() if mode == "row" else s_w.item(), g, io=io)
    assert np.array_equal(host_bits(wu), ref)


@pytest.mark.parametrize("io", ["bf16", "f16"])
@pytest.mark.parametrize("mode", ["tensor", "row"])
@pytest.mark.parametrize("M,N,K", [(1, 3, 128), (17, 1000, 384), (300, 1001, 1024), (700, 2048, 512)])
def test_default_linear_within_bound(io, mode, M, N, K):
    g = 128
    wq, s_w = prepared(N, K, g, mode, M * 3 + N)
    x = act(M, K, M + K, io)
    bias = f16_bits(np.random.default_rng(N).standard_normal(N) * 0.01) if io == "f16" else \
        synth.to_bf16_bits(np.random.default_rng(N).standard_normal(N) * 0.01)
    y = B.convrot_default_linear(dev16(x, io), wq, s_w, g, dev16(bias, io))
    wu = oracle.unpack_weight(wq.cpu().numpy(), s_w.cpu().numpy() if mode == "row" else s_w.item(), g, io=io)
    assert_default_close(host_bits(y), x, np.arange(M), wu, bias, io, K)


@pytest.mark.parametrize("tile", ["big", "big8", "wide", "wide128", "mid", "skinny", "skinny16", "half", "p128", "phalf", "tall", "ptall",
                                  "m32", "m64", "m128", "ksplit", "ksplit1536", "ksplit2048"])
def test_default_product_on_every_tile(tile, monkeypatch):
    monkeypatch.setenv("CONVROT_GEMM_TILE", tile[:6] if tile.startswith("ksplit") else tile)
    # the bf16 product runs the tiles with K counted in bytes: K = 1536 and
    # 2048 elements take the K-split tile's register-streamed form
    M, N, K, g = (11, 1001, int(tile[6:] or 640), 128) if tile.startswith("ksplit") else (300, 1001, 640, 128)
    wq, s_w = prepared(N, K, g, "tensor", 5)
    x = act(M, K, 6, "bf16")
    y = B.convrot_default_linear(dev16(x, "bf16"), wq, s_w, g, None)
    wu = oracle.unpack_weight(wq.cpu().numpy(), s_w.item(), g)
    assert_default_close(host_bits(y), x, np.arange(M), wu, None, "bf16", K)


def test_default_linear_at_the_bench_shape():
    # the whole 4608 x 3072 x 12288 layer, compared on 48 seeded token rows
    L = synth.make_layer("mlp_up")
    w = torch.from_numpy(L.w).to(DEV)
    wq, s_w = B.convrot_prepare_weight(w, L.g)
    y = B.convrot_default_linear(dev16(L.x_bits, "bf16"), wq, s_w, L.g, dev16(L.bias_bits, "bf16"))
    rows = synth.sample_rows(L.M, 48, 7)
    wu = oracle.unpack_weight(wq.cpu().numpy(), s_w.item(), L.g)
    assert_default_close(host_bits(y[torch.from_numpy(rows).to(DEV)]), L.x_bits, rows, wu, L.bias_bits,
                         "bf16", L.K)


# ---------------------------------------------------------------- guarded layer

@pytest.fixture
def guard():
    B.convrot_guard_configure(0.1, log_to_stderr=False)
    B.convrot_guard_reset(0)
    yield
    B.convrot_guard_reset(0)
    B.convrot_guard_configure(0.1, log_to_stderr=True)


def layer(M, N, K, g, io="bf16", mode="tensor", seed=1):
    wq, s_w = prepared(N, K, g, mode, seed)
    x = dev16(act(M, K, seed + 1, io), io)
    bias_np = np.random.default_rng(seed).standard_normal(N) * 0.01
    bias = dev16(f16_bits(bias_np) if io == "f16" else synth.to_bf16_bits(bias_np), io)
    return x, wq, s_w, bias


def same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("io,mode", [("bf16", "tensor"), ("f16", "row")])
def test_first_call_per_bucket_is_checked(guard, io, mode):
    g = 128
    x, wq, s_w, bias = layer(700, 1024, 3072, g, io, mode)
    y = B.convrot_linear_guarded(x, wq, s_w, g, bias)
    assert same(y, B.convrot_linear_ex(x, wq, s_w, g, bias))      # the int8 result, untouched
    st = B.convrot_guard_query(0)
    assert not st["fallback"] and st["checks_run"] == 1 and st["checked"] == 1
    assert 0.0 < st["last_error"] < 0.05
    assert "int8 matrix cores" in st["message"]
    # same bucket (M rounded up to 1024): no new check
    B.convrot_linear_guarded(x[:600], wq, s_w, g, bias)
    assert B.convrot_guard_query(0)["checks_run"] == 1
    # a new bucket: checked once
    x2, _, _, _ = layer(1100, 1024, 3072, g, io, mode, seed=1)
    y2 = B.convrot_linear_guarded(x2, wq, s_w, g, bias)
    assert same(y2, B.convrot_linear_ex(x2, wq, s_w, g, bias))
    assert B.convrot_guard_query(0)["checks_run"] == 2


@pytest.mark.parametrize("fault,words", [("mismatch", "does not match"), ("kernel", "failed")])
def test_fault_switches_the_device_to_the_default_path(guard, fault, words):
    g = 128
    x, wq, s_w, bias = layer(300, 2048, 1024, g)
    B.convrot_linear_guarded(x, wq, s_w, g, bias)          # checked, on the int8 path
    B.convrot_guard_inject(0, fault)
    y = B.convrot_linear_guarded(x, wq, s_w, g, bias)
    default = B.convrot_default_linear(x, wq, s_w, g, bias)
    assert same(y, default)
    st = B.convrot_guard_query(0)
    assert st["fallback"] and words in st["message"]
    # sticky: later calls, any bucket, take the default path with no new check
    runs = st["checks_run"]
    x3, _, _, _ = layer(5000, 2048, 1024, g, seed=1)
    assert same(B.convrot_linear_guarded(x3, wq, s_w, g, bias), B.convrot_default_linear(x3, wq, s_w, g, bias))
    assert B.convrot_guard_query(0)["checks_run"] == runs
    # until the state is reset
    B.convrot_guard_reset(0)
    assert same(B.convrot_linear_guarded(x, wq, s_w, g, bias), B.convrot_linear_ex(x, wq, s_w, g, bias))


def test_check_passes_on_the_page_workloads(guard):
    # the int8 layer differs from the default path by its activation
    # quantization only: well inside the tolerance on every workload shape
    for name in ("tiny", "qkv", "small_m", "stack_b0_out", "stack_b59_down"):
        L = synth.make_layer(name)
        w = torch.from_numpy(L.w).to(DEV)
        wq, s_w = B.convrot_prepare_weight(w, L.g)
        x, bias = dev16(L.x_bits, "bf16"), dev16(L.bias_bits, "bf16")
        y = B.convrot_linear_guarded(x, wq, s_w, L.g, bias)
        st = B.convrot_guard_query(0)
        assert not st["fallback"] and st["last_error"] < 0.05, (name, st)
        assert same(y, B.convrot_linear(x, wq, s_w, L.g, bias)), name
        B.convrot_guard_reset(0)


def test_checking_call_refuses_capture_then_graph_replays_after_it(guard):
    g = 128
    x, wq, s_w, bias = layer(512, 1024, 3072, g)
    y = torch.empty((512, 1024), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(B.convrot_guarded_workspace(512, 3072, 1024), dtype=torch.uint8, device=DEV)
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(B.ConvrotError) as e:
        with torch.cuda.graph(graph):
            B.convrot_linear_guarded(x, wq, s_w, g, bias, out=y, workspace=ws)
    assert "captured" in str(e.value)
    torch.cuda.synchronize()
    B.convrot_linear_guarded(x, wq, s_w, g, bias, out=y, workspace=ws)    # the check, eagerly
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.convrot_linear_guarded(x, wq, s_w, g, bias, out=y, workspace=ws)
    torch.cuda.synchronize()
    for _ in range(3):
        y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert same(y, B.convrot_linear(x, wq, s_w, g, bias))


def test_check_agrees_where_both_paths_overflow_fp16(guard):
    # one output channel past the fp16 range on both paths: a constant
    # activation of 100 (rotated exactly: one nonzero per group) against a
    # constant weight row of 0.1 gives ~10240, plus a bias of 60000; the
    # rounded output is +inf on the int8 layer and on the default path alike,
    # which is agreement, not a mismatch.  Every other channel is finite.
    M, N, K, g = 64, 256, 1024, 128
    w = weight(N, K, 11)
    w[5] = 0.1
    wq, s_w = B.convrot_prepare_weight_ex(torch.from_numpy(w).to(DEV), g, scale_mode="tensor")
    x = dev16(f16_bits(np.full((M, K), 100.0)), "f16")
    b = np.random.default_rng(3).standard_normal(N) * 0.01
    b[5] = 60000.0
    bias = dev16(f16_bits(b), "f16")
    y = B.convrot_linear_guarded(x, wq, s_w, g, bias)
    y_int8 = B.convrot_linear_ex(x, wq, s_w, g, bias)
    y_def = B.convrot_default_linear(x, wq, s_w, g, bias)
    assert torch.isinf(y_int8[:, 5]).all() and torch.isinf(y_def[:, 5]).all()
    assert torch.isfinite(y_int8[:, [c for c in range(N) if c != 5]]).all()
    st = B.convrot_guard_query(0)
    assert not st["fallback"] and st["checks_run"] == 1, st
    assert 0.0 <= st["last_error"] < 0.05
    assert same(y, y_int8)
