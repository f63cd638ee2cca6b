"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

* the library loads and exports every function include/convrot.h declares;
* argument errors are reported with the documented status before any launch
  (fake device addresses are passed: a call that got past its checks would
  touch them, so these tests also show that the checks come first);
* the workspace contract of the page "int8 Compute", section "Memory": the
  activation is coded a slice of tokens at a time, a slice holding no more
  tokens than two output widths, which keeps the working memory inside the
  2*N*K bytes that an unpacked bf16 weight would take.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convrot.h")

OK, EINVAL, EUNSUPPORTED, EALIGN, EWORKSPACE = 0, -1, -2, -3, -4
A = 0x10000          # a fake, 16-byte aligned device address (never dereferenced)


@pytest.fixture(scope="module")
def binding():
    from w8a8_rotated_int8_convrot_amd import binding, build
    if not os.path.exists(binding.LIB_PATH):
        build.build()
    binding.lib()
    return binding


@pytest.fixture(scope="module")
def lib(binding):
    return binding.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(convrot_\w+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("convrot_prepare_weight", "convrot_linear", "convrot_rotate_quant",
              "convrot_gemm_i32", "convrot_gemm_dequant", "convrot_last_error",
              "convrot_abi_version", "convrot_linear_workspace", "convrot_prepare_weight_workspace"):
        assert n in names


def test_library_exports_every_declared_symbol(lib, binding):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in binding.SIGNATURES, name
        assert hasattr(binding, name), name        # Python binding of the same name


def test_abi_version_matches_header(lib):
    m = re.search(r"#define\s+CONVROT_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert lib.convrot_abi_version() == int(m.group(1))


def facts():
    out = {}
    for line in open(os.path.join(ROOT, "tests", "golden", "pages_facts.txt")):
        line = line.split("#")[0].split()
        if line:
            out[line[0]] = float(line[1])
    return out


@pytest.mark.parametrize("M,K,N", [(4608, 3072, 12288), (4608, 12288, 3072), (16896, 3072, 12288),
                                   (16, 4096, 12288), (1000, 256, 96), (1, 128, 1)])
def test_workspace_stays_within_unpacked_weight(lib, M, K, N):
    per_width = facts()["slice_rows_per_output_width"]
    S = int(min(M, per_width * N))
    ws = lib.convrot_linear_workspace(M, K, N)
    assert ws >= S * K + 4 * S
    assert ws <= S * K + 4 * S + 256
    assert ws <= 2 * N * K + 4 * S + 256          # unpacked bf16 weight + the scales


def call_linear(lib, x=A, M=64, K=512, wq=A, ws_scale=A, N=64, g=128, bias=None, y=A,
                ws=A, ws_bytes=1 << 20):
    return lib.convrot_linear(x, M, K, wq, ws_scale, N, g, bias, y, ws, ws_bytes, None)


def test_linear_argument_errors(lib):
    assert call_linear(lib, g=64) == EUNSUPPORTED
    assert b"group" in lib.convrot_last_error()
    assert call_linear(lib, g=512) == EUNSUPPORTED
    assert call_linear(lib, K=384, g=256) == EINVAL          # K % group != 0
    assert call_linear(lib, K=131072 + 128) == EINVAL        # K too large for int32 sums
    assert call_linear(lib, N=0) == EINVAL
    assert call_linear(lib, M=-1) == EINVAL
    assert call_linear(lib, x=None) == EINVAL
    assert call_linear(lib, y=None) == EINVAL
    assert call_linear(lib, x=A + 8) == EALIGN
    assert call_linear(lib, y=A + 2) == EALIGN
    assert call_linear(lib, ws=A + 4) == EALIGN
    assert call_linear(lib, ws=None) == EWORKSPACE
    assert call_linear(lib, ws_bytes=15 * (512 + 4)) == EWORKSPACE   # less than one 16-row slice
    assert b"workspace" in lib.convrot_last_error()


def test_noalloc_argument_errors(lib):
    # refused before any HIP call, like convrot_linear (no workspace argument)
    f = lib.convrot_linear_noalloc
    assert f(A, 64, 512, A, A, 64, 64, None, A, None) == EUNSUPPORTED
    assert f(A, 64, 500, A, A, 64, 128, None, A, None) == EINVAL
    assert f(A, 64, 512, A, A, 0, 128, None, A, None) == EINVAL
    assert f(None, 64, 512, A, A, 64, 128, None, A, None) == EINVAL
    assert f(A + 8, 64, 512, A, A, 64, 128, None, A, None) == EALIGN
    assert f(A, 64, 512, A, A, 64, 128, None, A + 2, None) == EALIGN
    assert f(None, 0, 512, None, None, 64, 128, None, None, None) == OK
    assert lib.convrot_last_error() == b""


def test_empty_batch_needs_nothing(lib):
    assert call_linear(lib, M=0, x=None, y=None, ws=None, ws_bytes=0) == OK
    assert lib.convrot_last_error() == b""
    assert lib.convrot_rotate_quant(None, 0, 256, 128, None, None, None) == OK
    assert lib.convrot_gemm_dequant(None, None, None, None, None, None, 0, 4, 128, None) == OK


def test_stage_argument_errors(lib):
    assert lib.convrot_rotate_quant(A, 4, 512, 100, A, A, None) == EUNSUPPORTED
    assert lib.convrot_rotate_quant(A, 4, 640, 256, A, A, None) == EINVAL
    assert lib.convrot_rotate_quant(A + 1, 4, 512, 128, A, A, None) == EALIGN
    assert lib.convrot_gemm_i32(A, A, 4, 4, 100, A, None) == EINVAL          # K % 128
    assert lib.convrot_gemm_i32(A, A, 4, 4, 256, A + 4, None) == EALIGN
    assert lib.convrot_gemm_i32(A, None, 4, 4, 256, A, None) == EINVAL
    assert lib.convrot_gemm_dequant(A, A, A, A, None, A + 2, 4, 4, 256, None) == EALIGN
    assert lib.convrot_gemm_dequant(A, None, A, A, None, A, 4, 4, 256, None) == EINVAL


def test_prepare_weight_argument_errors(lib):
    f = lib.convrot_prepare_weight
    assert f(A, 7, 64, 512, 128, A, A, A, 256, None) == EUNSUPPORTED       # dtype
    assert f(A, 0, 64, 512, 64, A, A, A, 256, None) == EUNSUPPORTED        # group
    assert f(A, 0, 0, 512, 128, A, A, A, 256, None) == EINVAL
    assert f(A, 0, 64, 500, 128, A, A, A, 256, None) == EINVAL
    assert f(A, 0, 64, 512, 128, A, A, A, 2, None) == EWORKSPACE
    assert f(A, 0, 64, 512, 128, A, A, None, 256, None) == EWORKSPACE
    assert f(A + 4, 0, 64, 512, 128, A, A, A, 256, None) == EALIGN
    assert lib.convrot_prepare_weight_workspace(64, 512) >= 4


def test_binding_refuses_cpu_tensors(binding):
    import torch
    with pytest.raises(ValueError):
        binding.convrot_rotate_quant(torch.zeros((2, 128), dtype=torch.bfloat16), 128)


def test_mfma_probe_argument_errors(lib):
    f = lib.convrot_probe_mfma_i8
    assert f(A, 4096, A, 4096, 0, 10, A, None) == EINVAL          # no blocks
    assert f(A, 4096, A, 4096, 4, 0, A, None) == EINVAL           # no iterations
    assert f(A, 8, A, 4096, 4, 10, A, None) == EINVAL             # operand under 16 bytes
    assert f(None, 4096, A, 4096, 4, 10, A, None) == EINVAL
    assert f(A + 4, 4096, A, 4096, 4, 10, A, None) == EALIGN
    assert f(A, 4096, A, 4096, 4, 10, A + 8, None) == EALIGN
    assert b"aligned" in lib.convrot_last_error()


def test_stream_probe_argument_errors(lib):
    f = lib.convrot_probe_stream
    assert f(A, 12, A, None) == EINVAL                             # not a multiple of 8
    assert f(A, -8, A, None) == EINVAL
    assert f(None, 8, A, None) == EINVAL
    assert f(A + 4, 8, A, None) == EALIGN
    assert f(A, 8, A + 8, None) == EALIGN
    assert f(None, 0, None, None) == 0                             # n = 0: nothing to do


def test_variant_argument_errors(lib):
    F16 = 2
    # unknown io dtype / scale mode
    assert lib.convrot_rotate_quant_ex(A, 7, 4, 512, 128, A, A, None) == EUNSUPPORTED
    assert lib.convrot_gemm_dequant_ex(A, A, A, A, 2, None, A, 1, 4, 4, 256, None) == EUNSUPPORTED
    assert lib.convrot_gemm_dequant_ex(A, A, A, A, 0, None, A, 0, 4, 4, 256, None) == EUNSUPPORTED
    assert lib.convrot_linear_ex(A, F16, 64, 512, A, A, 5, 64, 128, None, A, A, 1 << 20, None) == EUNSUPPORTED
    assert lib.convrot_prepare_weight_ex(A, 0, 64, 512, 128, 3, A, A, A, 256, None) == EUNSUPPORTED
    # fp16 weights go through the _ex entry point only
    assert lib.convrot_prepare_weight(A, F16, 64, 512, 128, A, A, A, 256, None) == EUNSUPPORTED
    assert b"_ex" in lib.convrot_last_error()
    # the rules of the plain entry points still apply
    assert lib.convrot_linear_ex(A, F16, 64, 500, A, A, 1, 64, 128, None, A, A, 1 << 20, None) == EINVAL
    assert lib.convrot_linear_ex(A + 2, F16, 64, 512, A, A, 1, 64, 128, None, A, A, 1 << 20, None) == EALIGN
    assert lib.convrot_gemm_dequant_ex(A, A, A, A, 1, None, A + 4, F16, 4, 4, 256, None) == EALIGN
    assert lib.convrot_linear_ex(None, F16, 0, 512, None, None, 1, 64, 128, None, None, None, 0, None) == OK


def test_streamed_argument_errors(lib, binding):
    import ctypes
    L = binding.StreamLayer(A, 64, 512, 64, A, A, 128, None, A)
    arr = (binding.StreamLayer * 2)(L, L)
    f = lib.convrot_linear_streamed
    assert f(None, 2, A, 1 << 16, A, 1 << 20, None, None) == EINVAL
    assert f(arr, -1, A, 1 << 16, A, 1 << 20, None, None) == EINVAL
    assert f(arr, 0, None, 0, None, 0, None, None) == OK
    assert f(arr, 2, A + 8, 1 << 16, A, 1 << 20, None, None) == EALIGN
    assert f(arr, 2, A, 1024, A, 1 << 20, None, None) == EWORKSPACE          # slot < N*K
    assert f(arr, 2, A, 1 << 16, A, 100, None, None) == EWORKSPACE            # workspace
    bad = (binding.StreamLayer * 1)(binding.StreamLayer(A, 64, 512, 64, A, A, 64, None, A))
    assert f(bad, 1, A, 1 << 16, A, 1 << 20, None, None) == EUNSUPPORTED       # group
    assert lib.convrot_stream_slot_bytes(arr, 2) == 64 * 512
    assert ctypes.sizeof(binding.StreamLayer) == 72


def test_default_path_and_guard_argument_errors(lib):
    F16, BF16 = 2, 1
    big = 1 << 30
    # default path: the layer rules, and a workspace of at least the unpacked weight
    assert lib.convrot_default_workspace(512, 64) == 2 * 512 * 64
    assert lib.convrot_default_linear(A, BF16, 64, 512, A, A, 0, 64, 128, None, A, A, 2 * 512 * 64 - 1,
                                      None) == EWORKSPACE
    assert lib.convrot_default_linear(A, BF16, 64, 500, A, A, 0, 64, 128, None, A, A, big, None) == EINVAL
    assert lib.convrot_default_linear(A, BF16, 64, 512, A, A, 0, 64, 96, None, A, A, big, None) == EUNSUPPORTED
    assert lib.convrot_default_linear(A, 0, 64, 512, A, A, 0, 64, 128, None, A, A, big, None) == EUNSUPPORTED
    assert lib.convrot_default_linear(A + 2, F16, 64, 512, A, A, 0, 64, 128, None, A, A, big, None) == EALIGN
    assert lib.convrot_default_linear(None, BF16, 0, 512, None, None, 0, 64, 128, None, None, None, 0,
                                      None) == OK
    assert lib.convrot_unpack_weight(A, A, 0, 64, 512, 128, 0, A, None) == EUNSUPPORTED   # fp32 out
    assert lib.convrot_unpack_weight(A, A, 2, 64, 512, 128, BF16, A, None) == EUNSUPPORTED
    assert lib.convrot_unpack_weight(A, None, 0, 64, 512, 128, BF16, A, None) == EINVAL
    assert lib.convrot_unpack_weight(A, A, 0, 64, 512, 128, BF16, A + 8, None) == EALIGN
    # guarded layer: the same rules, and its own workspace
    ws = lib.convrot_guarded_workspace(64, 512, 64)
    assert lib.convrot_linear_guarded(A, BF16, 64, 512, A, A, 0, 64, 128, None, A, A, ws - 1, None) == EWORKSPACE
    assert lib.convrot_linear_guarded(A, BF16, 64, 512, A, A, 3, 64, 128, None, A, A, ws, None) == EUNSUPPORTED
    assert lib.convrot_linear_guarded(A, BF16, 64, 512, A, A, 0, 0, 128, None, A, A, ws, None) == EINVAL
    assert lib.convrot_linear_guarded(None, BF16, 0, 512, None, None, 0, 64, 128, None, None, None, 0,
                                      None) == OK


@pytest.mark.parametrize("M,K,N", [(1, 128, 1), (300, 512, 64), (4608, 3072, 12288), (16, 4096, 12288)])
def test_guarded_workspace_is_the_unpacked_weight_plus_the_kept_rows(lib, M, K, N):
    # page "int8 Compute", "Memory": the default path reserves the unpacked
    # weight; the check keeps 256 rows of the output from each path (here also
    # the 256 gathered activation rows and three fp64 sums per row)
    R = min(M, 256)
    pad = lambda v: (v + 255) // 256 * 256
    ws = lib.convrot_guarded_workspace(M, K, N)
    assert ws >= lib.convrot_linear_workspace(M, K, N)
    assert ws == max(lib.convrot_linear_workspace(M, K, N),
                     pad(2 * N * K) + pad(2 * R * K) + pad(2 * R * N) + pad(24 * R))


def test_guard_state_on_the_host(lib, binding):
    # state functions touch no device
    binding.convrot_guard_reset(5)
    st = binding.convrot_guard_query(5)
    assert st == {"fallback": False, "checked": 0, "checks_run": 0, "last_error": -1.0, "message": ""}
    binding.convrot_guard_inject(5, "mismatch")
    binding.convrot_guard_inject(5, "none")
    binding.convrot_guard_reset(5)
    assert lib.convrot_guard_inject(5, 9) == EINVAL
    assert lib.convrot_guard_inject(-1, 1) == EINVAL
    assert lib.convrot_guard_query(0, None) == EINVAL
    assert lib.convrot_guard_reset(-2) == EINVAL
    assert lib.convrot_guard_configure(0.0, 1) == EINVAL
    assert lib.convrot_guard_configure(float("nan"), 1) == EINVAL
    assert lib.convrot_guard_configure(float("inf"), 1) == EINVAL
    assert lib.convrot_guard_configure(0.1, 1) == OK
    with pytest.raises(ValueError):
        binding.convrot_guard_inject(0, "segfault")
    assert ctypes.sizeof(binding.GuardInfo) == 288


def test_token_row_multiply_shift_is_exact():
    """The token-block rotate kernel finds a lane's token row as
    (b * ceil(2^16 / bpr)) >> 16 instead of b / bpr, for block index
    b < 256 (two lanes per block, at most 512 lanes) and bpr = K / 128 <= 256
    blocks per row (K <= 32768 on that kernel).  Exact for every such pair,
    and every product fits the 24-bit multiplier it uses."""
    for bpr in range(1, 257):
        inv = (65536 + bpr - 1) // bpr
        for b in range(256):
            assert b * inv < (1 << 24)
            assert (b * inv) >> 16 == b // bpr, (b, bpr)
