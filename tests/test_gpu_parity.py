"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: int8 codes, scales and int32 products bit-exact; bf16 outputs within
relative Frobenius error 1e-2 of the oracle (and bit-exact where the oracle's
own int8/int32 tensors are fed to the epilogue).  Full-size workloads are run
whole on the GPU and compared on seeded sampled token rows, which the oracle
evaluates one by one (each token is quantized on its own, so a sampled row of
the layer is exactly that row of the full result); weights and scales are
compared in full.
"""
import numpy as np
import pytest
import torch

import oracle
from tests._util import bits_of, rel_frobenius, same_bf16, to_dev_bf16
from w8a8_rotated_int8_convrot_amd import synth

pytestmark = pytest.mark.gpu

REL_TOL = 1e-2          # bf16 output vs oracle, relative Frobenius
NRMSE_GATE = 0.05       # quantized output vs unquantized fp64 product


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from w8a8_rotated_int8_convrot_amd import binding
    binding.lib()
    return binding


DEV = "cuda:0"


def rand_bf16(M, K, seed, outliers=4, factor=20.0):
    r = np.random.default_rng(seed)
    x = r.standard_normal((M, K))
    if outliers:
        x[:, r.choice(K, outliers, replace=False)] *= factor
    return synth.to_bf16_bits(x)


# ---------------------------------------------------------------- rotate + quant

# Batches of up to 2^21 elements with K < 8192 take the row kernel (a row
# spread over 256 lanes); larger batches, or K >= 8192, with K <= 32768 the
# block kernel (two lanes per 128 elements, several rows per workgroup);
# K > 32768 the row kernel in two passes.
ROTQ_CASES = [
    (5, 128, 128), (131, 512, 128), (300, 3072, 128), (77, 3072, 256), (40, 4096, 128),
    (33, 12288, 128), (20, 12288, 256), (9, 16384, 128), (7, 24576, 256), (3, 131072, 128),
    (701, 3072, 128), (523, 4096, 256), (171, 12288, 128), (129, 16384, 256), (67, 32768, 128),
    (600, 12288, 128), (1024, 3072, 256),
    (3, 33024, 256), (2, 33280, 128),          # two-pass rows with a partial last segment
]


@pytest.mark.parametrize("M,K,g", ROTQ_CASES)
def test_rotate_quant_bit_exact(B, M, K, g):
    x = rand_bf16(M, K, seed=M * 7 + K + g)
    x[0] = 0                                   # a zero token
    if M > 2:
        x[1] = 0
        x[1, K // 3] = synth.to_bf16_bits(np.array([-3.0]))[0]   # a one-hot token
    q, s = B.convrot_rotate_quant(to_dev_bf16(x, DEV), g)
    q_ref, s_ref = oracle.quant_act(x, g)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy(), s_ref)


# ---------------------------------------------------------------- weights

@pytest.mark.parametrize("N,K,g,dt", [(512, 512, 128, "f32"), (300, 3072, 256, "f32"),
                                      (1000, 384, 128, "bf16"), (7, 16384, 128, "f32"),
                                      (33, 12288, 256, "bf16"), (5, 13056, 256, "f32")])
def test_prepare_weight_bit_exact(B, N, K, g, dt):
    r = np.random.default_rng(N + K)
    w = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[N // 2, K // 5] = 0.9                    # one large weight sets the tensor scale
    if dt == "bf16":
        wb = synth.to_bf16_bits(w)
        w = oracle.bf16_bits_to_f32(wb)
        wt = to_dev_bf16(wb, DEV)
    else:
        wt = torch.from_numpy(w).to(DEV)
    wq, s = B.convrot_prepare_weight(wt, g)
    wq_ref, s_ref = oracle.quant_weight(w, g)
    assert np.array_equal(wq.cpu().numpy(), wq_ref)
    assert s.item() == float(s_ref)


def test_prepare_weight_zero(B):
    wq, s = B.convrot_prepare_weight(torch.zeros((64, 256), device=DEV), 128)
    assert s.item() == 0.0 and int(wq.abs().max()) == 0


# ---------------------------------------------------------------- GEMM stages

GEMM_CASES = [(1, 1, 128), (17, 33, 256), (300, 200, 384), (513, 1000, 1024), (64, 12288, 4096),
              (2304, 2560, 640), (4608, 12288, 3072)]


def rand_i8(shape, seed):
    return np.random.default_rng(seed).integers(-127, 128, size=shape, dtype=np.int64).astype(np.int8)


@pytest.mark.parametrize("M,N,K", GEMM_CASES)
def test_gemm_i32_bit_exact(B, M, N, K):
    a = rand_i8((M, K), M + 3 * N + K)
    b = rand_i8((N, K), M * N + K)
    acc = B.convrot_gemm_i32(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV))
    rows = synth.sample_rows(M, 48, M + N) if M * N * K > 2e9 else np.arange(M)
    got = acc[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    assert np.array_equal(got, oracle.gemm_i32(a[rows], b))


def test_gemm_i32_extreme_accumulators(B):
    K = 131072
    a = np.full((3, K), 127, np.int8)
    a[1] = -127
    b = np.full((5, K), 127, np.int8)
    b[2] = -127
    b[4, ::2] = -127
    acc = B.convrot_gemm_i32(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV)).cpu().numpy()
    assert np.array_equal(acc, oracle.gemm_i32(a, b))
    assert acc[0, 0] == 127 * 127 * K


@pytest.mark.parametrize("M,N,K", [(17, 33, 256), (300, 1001, 384), (513, 1000, 1024), (4608, 12288, 3072)])
@pytest.mark.parametrize("with_bias", [True, False])
def test_gemm_dequant_bit_exact(B, M, N, K, with_bias):
    r = np.random.default_rng(M + N)
    a = rand_i8((M, K), M + N + K)
    b = rand_i8((N, K), 3 * M + N)
    s_x = (r.random(M) * 0.2 + 1e-3).astype(np.float32)
    s_w = np.float32(2.3e-4)
    bias = synth.to_bf16_bits(r.standard_normal(N) * 0.01) if with_bias else None
    y = B.convrot_gemm_dequant(torch.from_numpy(a).to(DEV), torch.from_numpy(s_x).to(DEV),
                               torch.from_numpy(b).to(DEV), torch.tensor([s_w], device=DEV),
                               None if bias is None else to_dev_bf16(bias, DEV))
    rows = synth.sample_rows(M, 48, M) if M * N * K > 2e9 else np.arange(M)
    got = bits_of(y[torch.from_numpy(rows).to(DEV)])
    ref = oracle.epilogue(oracle.gemm_i32(a[rows], b), s_x[rows], s_w, bias)
    assert np.all(same_bf16(got, ref))


# ---------------------------------------------------------------- whole layer

E2E = [("tiny", 128), ("tiny", 256), ("qkv", 128), ("mlp_up", 128), ("mlp_up", 256),
       ("mlp_down", 128), ("hires_up", 128), ("small_m", 128),
       ("stack_b0_qkv", 128), ("stack_b0_out", 128), ("stack_b59_up", 128), ("stack_b59_down", 128)]


def run_layer(B, L):
    x = to_dev_bf16(L.x_bits, DEV)
    w = torch.from_numpy(L.w).to(DEV)
    bias = to_dev_bf16(L.bias_bits, DEV)
    wq, s_w = B.convrot_prepare_weight(w, L.g)
    y = B.convrot_linear(x, wq, s_w, L.g, bias)
    q, s = B.convrot_rotate_quant(x, L.g)
    return x, wq, s_w, bias, y, q, s


@pytest.mark.parametrize("name,g", E2E)
def test_linear_end_to_end(B, name, g):
    L = synth.make_layer(name, g=g)
    x, wq, s_w, bias, y, q, s = run_layer(B, L)
    torch.cuda.synchronize()

    wq_ref, s_w_ref = oracle.quant_weight(L.w, L.g)
    assert np.array_equal(wq.cpu().numpy(), wq_ref), "weight codes"
    assert s_w.item() == float(s_w_ref), "weight scale"

    # 256 seeded rows for the 2048^2 layer and the stack, 64 for the others
    count = 256 if name.startswith(("hires", "stack")) else 64
    rows = np.arange(L.M) if L.M <= 256 else synth.sample_rows(L.M, count, L.M + L.N)
    y_ref, q_ref, s_ref = oracle.linear_rows(L.x_bits, rows, wq_ref, s_w_ref, L.g, L.bias_bits)
    ridx = torch.from_numpy(rows).to(DEV)
    q_gpu = q[ridx].cpu().numpy()
    # activation codes: bit-exact (and therefore 100 % identical, none off by > 1)
    assert np.array_equal(q_gpu, q_ref), f"codes differ at {np.argwhere(q_gpu != q_ref)[:5]}"
    assert np.array_equal(s[ridx].cpu().numpy(), s_ref), "token scales"

    y_gpu = bits_of(y[ridx])
    assert np.all(np.isfinite(oracle.bf16_bits_to_f32(y_gpu)))
    err = rel_frobenius(y_gpu, y_ref)
    assert err <= REL_TOL, f"rel-Frobenius {err}"
    # with identical codes the epilogue is deterministic: expect every value equal
    assert np.mean(same_bf16(y_gpu, y_ref)) == 1.0

    # sanity gate against the unquantized product
    ref64 = oracle.reference_fp64(L.x_bits[rows], L.w, L.bias_bits)
    assert oracle.nrmse(oracle.bf16_bits_to_f32(y_gpu), ref64) <= NRMSE_GATE


# ---------------------------------------------------------------- invariances and edges

def test_result_does_not_depend_on_slicing(B):
    L = synth.make_layer("tiny")
    x, wq, s_w, bias, y, _, _ = run_layer(B, L)
    full = bits_of(y)
    for rows in (16, 48, 112):
        ws = torch.empty(rows * L.K + 256 + rows * 4, dtype=torch.uint8, device=DEV)
        y2 = B.convrot_linear(x, wq, s_w, L.g, bias, workspace=ws)
        assert np.array_equal(bits_of(y2), full), rows


def test_slicing_at_twice_the_output_width(B):
    # M > 2N: the default workspace holds 2N tokens, so the call runs in slices
    r = np.random.default_rng(4)
    M, K, N = 1000, 256, 96
    xb = rand_bf16(M, K, 5)
    w = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    x = to_dev_bf16(xb, DEV)
    wq, s_w = B.convrot_prepare_weight(torch.from_numpy(w).to(DEV), 128)
    assert B.convrot_linear_workspace(M, K, N) < M * K
    y = B.convrot_linear(x, wq, s_w, 128)
    wq_ref, s_ref = oracle.quant_weight(w, 128)
    y_ref, _, _ = oracle.linear(xb, wq_ref, s_ref, 128)
    assert np.all(same_bf16(bits_of(y), y_ref))


def test_bit_identical_run_to_run(B):
    L = synth.make_layer("qkv", M=1024)
    x, wq, s_w, bias, y, q, s = run_layer(B, L)
    y2 = B.convrot_linear(x, wq, s_w, L.g, bias)
    q2, s2 = B.convrot_rotate_quant(x, L.g)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(q, q2) and torch.equal(s, s2)


# few-token shapes on each automatic choice: 16 x 16 (M <= 16), 64 x 64 and
# 64 x 128 (many channels), 32 x 32 and 64 x 32 (few channels, ragged N), and
# past 128 tokens 64 x 128 on layers too small for larger tiles (N down to 1),
# and 384 x 96 where 384 x 192 tiles would fill 3/8 to 1/2 of the CUs
@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (1, 3, 256), (2, 5, 128), (16, 12288, 4096), (63, 130, 512),
                                   (40, 12288, 1024), (100, 9216, 512), (64, 3072, 1536), (128, 3000, 384),
                                   (100, 1, 128), (65, 7, 256), (129, 5, 128), (300, 1001, 384),
                                   (3072, 3000, 256)])
def test_small_and_ragged_shapes(B, M, N, K):
    r = np.random.default_rng(M + N + K)
    xb = rand_bf16(M, K, M + K, outliers=0)
    w = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    bias = synth.to_bf16_bits(r.standard_normal(N) * 0.01)
    wq, s_w = B.convrot_prepare_weight(torch.from_numpy(w).to(DEV), 128)
    y = B.convrot_linear(to_dev_bf16(xb, DEV), wq, s_w, 128, to_dev_bf16(bias, DEV))
    wq_ref, s_ref = oracle.quant_weight(w, 128)
    y_ref, _, _ = oracle.linear(xb, wq_ref, s_ref, 128, bias)
    assert np.all(same_bf16(bits_of(y), y_ref))


# The few-token tiles (M <= 16): the one that splits K over its four waves
# and the one-wave tile; K from one slab (three waves of the K-split tile
# without work) to 96 slabs with uneven shares, ragged N, one token to
# sixteen, and K = 3072 and 4096, where the K-split tile streams its operands
# through registers; int32 and the bf16 epilogue against the oracle.
@pytest.mark.parametrize("tile", ["ksplit", "skinny16"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (7, 1000, 384), (16, 12289, 4096), (13, 3001, 12288),
                                   (16, 64, 640), (2, 12288, 1152), (5, 12290, 3072), (16, 33, 4096),
                                   (1, 17, 3072)])
def test_few_token_tiles_bit_exact(B, tile, M, N, K, monkeypatch):
    monkeypatch.setenv("CONVROT_GEMM_TILE", tile)
    r = np.random.default_rng(M * N + K)
    a = rand_i8((M, K), 3 * M + K)
    b = rand_i8((N, K), 5 * N + K)
    s_x = (r.random(M) * 0.2 + 1e-3).astype(np.float32)
    s_w = np.float32(1.3e-4)
    bias = synth.to_bf16_bits(r.standard_normal(N) * 0.01)
    ad, bd = torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV)
    acc = B.convrot_gemm_i32(ad, bd).cpu().numpy()
    y = B.convrot_gemm_dequant(ad, torch.from_numpy(s_x).to(DEV), bd, torch.tensor([s_w], device=DEV),
                               to_dev_bf16(bias, DEV))
    acc_ref = oracle.gemm_i32(a, b)
    assert np.array_equal(acc, acc_ref)
    assert np.all(same_bf16(bits_of(y), oracle.epilogue(acc_ref, s_x, s_w, bias)))


def test_empty_batch_is_a_no_op(B):
    wq = torch.zeros((8, 128), dtype=torch.int8, device=DEV)
    s_w = torch.ones(1, device=DEV)
    x = torch.empty((0, 128), dtype=torch.bfloat16, device=DEV)
    y = B.convrot_linear(x, wq, s_w, 128)
    assert y.shape == (0, 8)


@pytest.mark.parametrize("tile", ["big", "big8", "wide", "wide128", "mid", "skinny", "skinny16", "half", "p128", "phalf", "tall", "ptall",
                                  "m32", "m64", "m128"])
@pytest.mark.parametrize("M,N,K", [(300, 1001, 384), (513, 1000, 1024), (1111, 777, 640)])
def test_every_gemm_tile_is_bit_exact(B, tile, M, N, K, monkeypatch):
    # the tile shape is a performance choice: every one must give the same bytes
    monkeypatch.setenv("CONVROT_GEMM_TILE", tile)
    r = np.random.default_rng(M + N + K)
    a = rand_i8((M, K), 5 * M + K)
    b = rand_i8((N, K), 7 * N + K)
    s_x = (r.random(M) * 0.2 + 1e-3).astype(np.float32)
    s_w = np.float32(1.1e-4)
    bias = synth.to_bf16_bits(r.standard_normal(N) * 0.01)
    ad, bd = torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV)
    acc = B.convrot_gemm_i32(ad, bd).cpu().numpy()
    y = B.convrot_gemm_dequant(ad, torch.from_numpy(s_x).to(DEV), bd, torch.tensor([s_w], device=DEV),
                               to_dev_bf16(bias, DEV))
    acc_ref = oracle.gemm_i32(a, b)
    assert np.array_equal(acc, acc_ref)
    assert np.all(same_bf16(bits_of(y), oracle.epilogue(acc_ref, s_x, s_w, bias)))


@pytest.mark.parametrize("tile", ["p128", "ptall"])
@pytest.mark.parametrize("M,N,K", [(2500, 9001, 384), (3001, 12288, 640), (4608, 9216, 3072), (4608, 3072, 12288),
                                   (5000, 12289, 1152)])
def test_persistent_tiles_bit_exact(B, tile, M, N, K, monkeypatch):
    # the persistent 384 x 192 and 192 x 288 kernels with several tiles per
    # workgroup (the pipeline crosses tile boundaries), ragged edges, 3 to 24
    # slabs of K; with p128 the 4608 x 9216 layer also runs its 384 x 96
    # tail; int32 and the bf16 epilogue against the oracle on seeded rows,
    # which include the edges
    monkeypatch.setenv("CONVROT_GEMM_TILE", tile)
    a = rand_i8((M, K), 3 * M + K)
    b = rand_i8((N, K), 5 * N + K)
    r = np.random.default_rng(M + N + K)
    s_x = (r.random(M) * 0.2 + 1e-3).astype(np.float32)
    s_w = np.float32(1.1e-4)
    bias = synth.to_bf16_bits(r.standard_normal(N) * 0.01)
    ad, bd = torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV)
    acc = B.convrot_gemm_i32(ad, bd)
    y = B.convrot_gemm_dequant(ad, torch.from_numpy(s_x).to(DEV), bd, torch.tensor([s_w], device=DEV),
                               to_dev_bf16(bias, DEV))
    rows = synth.sample_rows(M, 40, M * 3 + N)
    ridx = torch.from_numpy(rows).to(DEV)
    acc_ref = oracle.gemm_i32(a[rows], b)
    assert np.array_equal(acc[ridx].cpu().numpy(), acc_ref)
    assert np.all(same_bf16(bits_of(y[ridx]), oracle.epilogue(acc_ref, s_x[rows], s_w, bias)))


@pytest.mark.parametrize("M", [2000, 2112])
def test_half_height_tail_split(B, M):
    # M = 2000 or 2112, N = 12288: 352 tiles of 384 x 192 would leave the second
    # round 96 of 256 full, so token rows [0, 1536) run as 384 x 192 tiles and
    # the rest as 384 x 96 tiles (ragged for M = 2000) in a second launch;
    # rows on both sides of the split and at the end are compared
    N, K = 12288, 384
    a = rand_i8((M, K), M)
    b = rand_i8((N, K), 3)
    r = np.random.default_rng(M)
    s_x = (r.random(M) * 0.2 + 1e-3).astype(np.float32)
    s_w = np.float32(1.3e-4)
    bias = synth.to_bf16_bits(r.standard_normal(N) * 0.01)
    ad, bd = torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV)
    acc = B.convrot_gemm_i32(ad, bd)
    y = B.convrot_gemm_dequant(ad, torch.from_numpy(s_x).to(DEV), bd, torch.tensor([s_w], device=DEV),
                               to_dev_bf16(bias, DEV))
    rows = np.unique(np.concatenate([[0, 191, 192, 1535, 1536, 1537, 1631, 1632, M - 2, M - 1],
                                     r.choice(M, 24, replace=False)]))
    ridx = torch.from_numpy(rows).to(DEV)
    acc_ref = oracle.gemm_i32(a[rows], b)
    assert np.array_equal(acc[ridx].cpu().numpy(), acc_ref)
    assert np.all(same_bf16(bits_of(y[ridx]), oracle.epilogue(acc_ref, s_x[rows], s_w, bias)))


@pytest.mark.parametrize("reps", [1, 700])       # row kernel; block kernel (M*K > 2^21)
def test_rotate_quant_exact_ties(B, reps):
    # g = 256 rotates exactly (1/sqrt(256) = 1/16): with x = H u the rotated
    # row is 16 u, so with max |u| = 127 the quotient v/s is u itself, and
    # half-integer entries of u land exactly on rounding ties of the code
    # (round half to even).  A third entry 0.5 keeps every x = H u entry an
    # integer or half-integer with at most 8 significant bits (exact in bf16).
    # The kernel's reciprocal fast path must hand ties to the exact division.
    g = 256
    H = oracle.hadamard(g).astype(np.float64)
    halves = (1.5, 2.5, -3.5, 62.5, -126.5, 0.5)
    rows = []
    for half in halves:
        u = np.zeros(g)
        u[0], u[7], u[9] = 127.0, half, 0.5
        rows.append(H @ u)
    xf = np.tile(np.array(rows), (reps, 2))
    x = synth.to_bf16_bits(xf)
    assert np.array_equal(oracle.bf16_bits_to_f32(x), xf.astype(np.float32))
    q, s = B.convrot_rotate_quant(to_dev_bf16(x, DEV), g)
    q_ref, s_ref = oracle.quant_act(x, g)
    assert np.array_equal(q.cpu().numpy(), q_ref) and np.array_equal(s.cpu().numpy(), s_ref)
    assert [int(q_ref[i, 7]) for i in range(len(halves))] == [2, 2, -4, 62, -126, 0]
    assert all(int(q_ref[i, 9]) == 0 for i in range(len(halves)))


# Seeded random shapes over every automatic tile choice (few tokens with many
# or few channels, 128 x 128 / 64 x 128 for small layers, 384 x 192 with and
# without its half-height tail, 256 x 256), ragged in M and N: int32 products
# bit-exact, the dequant epilogue bit-exact on the oracle's int32.
def _random_shapes(n, seed):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        band = i % 4
        if band == 0:
            M, N = int(r.integers(1, 17)), int(r.integers(1, 13000))
        elif band == 1:
            M, N = int(r.integers(17, 129)), int(r.integers(1, 13000))
        elif band == 2:
            M, N = int(r.integers(129, 1200)), int(r.integers(1, 4000))
        else:
            M, N = int(r.integers(1200, 3000)), int(r.integers(6000, 13000))
        K = 128 * int(r.integers(1, 2 if M * N > 8e6 else 5 if M * N > 4e6 else 17))
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", _random_shapes(16, 2026))
def test_random_shapes_bit_exact(B, M, N, K):
    a = rand_i8((M, K), M * 7 + K)
    b = rand_i8((N, K), N * 5 + K)
    r = np.random.default_rng(M + N)
    s_x = (r.random(M) * 0.2 + 1e-3).astype(np.float32)
    s_w = np.float32(1.7e-4)
    bias = synth.to_bf16_bits(r.standard_normal(N) * 0.01)
    ad, bd = torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV)
    acc = B.convrot_gemm_i32(ad, bd).cpu().numpy()
    y = B.convrot_gemm_dequant(ad, torch.from_numpy(s_x).to(DEV), bd, torch.tensor([s_w], device=DEV),
                               to_dev_bf16(bias, DEV))
    acc_ref = oracle.gemm_i32(a, b)
    assert np.array_equal(acc, acc_ref)
    assert np.all(same_bf16(bits_of(y), oracle.epilogue(acc_ref, s_x, s_w, bias)))


def _random_persistent(n, seed):
    r = np.random.default_rng(seed)
    return [(int(r.integers(1800, 6000)), int(r.integers(2000, 13000)), 128 * int(r.integers(3, 13)))
            for _ in range(n)]


# Seeded random shapes on the persistent kernels (several tiles per workgroup,
# ragged in M and N, 3 to 12 slabs of K): int32 and the bf16 epilogue against
# the oracle on seeded rows, which include the first and last.
@pytest.mark.parametrize("tile", ["p128", "ptall"])
@pytest.mark.parametrize("M,N,K", _random_persistent(6, 4242))
def test_random_persistent_shapes_bit_exact(B, tile, M, N, K, monkeypatch):
    monkeypatch.setenv("CONVROT_GEMM_TILE", tile)
    a = rand_i8((M, K), 11 * M + K)
    b = rand_i8((N, K), 13 * N + K)
    r = np.random.default_rng(M * N + K)
    s_x = (r.random(M) * 0.2 + 1e-3).astype(np.float32)
    s_w = np.float32(1.2e-4)
    bias = synth.to_bf16_bits(r.standard_normal(N) * 0.01)
    ad, bd = torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV)
    acc = B.convrot_gemm_i32(ad, bd)
    y = B.convrot_gemm_dequant(ad, torch.from_numpy(s_x).to(DEV), bd, torch.tensor([s_w], device=DEV),
                               to_dev_bf16(bias, DEV))
    rows = synth.sample_rows(M, 24, M + N)
    ridx = torch.from_numpy(rows).to(DEV)
    acc_ref = oracle.gemm_i32(a[rows], b)
    assert np.array_equal(acc[ridx].cpu().numpy(), acc_ref)
    assert np.all(same_bf16(bits_of(y[ridx]), oracle.epilogue(acc_ref, s_x[rows], s_w, bias)))


def _random_few(n, seed):
    r = np.random.default_rng(seed)
    return [(int(r.integers(1, 17)), int(r.integers(8192, 16000)), 128 * int(r.integers(1, 40)))
            for _ in range(n)]


# Seeded random few-token shapes on the automatic choice, which is the K-split
# tile for N / 16 >= 512 (every shape here): the whole int32 product and the
# bf16 epilogue against the oracle.
@pytest.mark.parametrize("M,N,K", _random_few(8, 1717))
def test_random_few_token_shapes_bit_exact(B, M, N, K):
    a = rand_i8((M, K), 17 * M + K)
    b = rand_i8((N, K), 19 * N + K)
    r = np.random.default_rng(M + N * K)
    s_x = (r.random(M) * 0.2 + 1e-3).astype(np.float32)
    s_w = np.float32(0.9e-4)
    bias = synth.to_bf16_bits(r.standard_normal(N) * 0.01)
    ad, bd = torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV)
    acc = B.convrot_gemm_i32(ad, bd).cpu().numpy()
    y = B.convrot_gemm_dequant(ad, torch.from_numpy(s_x).to(DEV), bd, torch.tensor([s_w], device=DEV),
                               to_dev_bf16(bias, DEV))
    acc_ref = oracle.gemm_i32(a, b)
    assert np.array_equal(acc, acc_ref)
    assert np.all(same_bf16(bits_of(y), oracle.epilogue(acc_ref, s_x, s_w, bias)))


def _random_rotq(n, seed):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        g = 128 if i % 3 else 256
        K = g * int(r.integers(1, 32768 // g + 1)) if i % 4 else g * int(r.integers(1, 8))
        M = int(r.integers(1, max(2, min(3000, (1 << 23) // K))))
        out.append((M, K, g))
    return out


@pytest.mark.parametrize("M,K,g", _random_rotq(12, 77))
def test_random_rotate_quant_bit_exact(B, M, K, g):
    # seeded random batch shapes over both activation kernels (small batches
    # with short rows on the row kernel, the rest on the token-block kernel)
    x = rand_bf16(M, K, seed=M + K + g, outliers=min(4, K // 64))
    q, s = B.convrot_rotate_quant(to_dev_bf16(x, DEV), g)
    q_ref, s_ref = oracle.quant_act(x, g)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy(), s_ref)
