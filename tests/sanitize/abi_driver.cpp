// abi_driver.cpp -- drives the argument checks of every C ABI entry point
// that can be reached without a GPU, for a host build of the library under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Every call here must be
// refused (or be a no-op such as M = 0) before any HIP call: the pointers are
// fake device addresses that nothing may dereference.  Exit status 0 and the
// line "abi_driver: N checks passed" mean every status matched.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/convrot.h"

static int g_checks = 0, g_failed = 0;

static void expect(int got, int want, const char* what) {
  ++g_checks;
  if (got != want) {
    ++g_failed;
    std::printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, convrot_last_error());
  } else if (got != CONVROT_OK && std::strlen(convrot_last_error()) == 0) {
    ++g_failed;
    std::printf("FAIL %s: status %d without a message\n", what, got);
  }
}

int main() {
  // fake, 256-byte aligned device addresses (never dereferenced) and a
  // misaligned one
  void* A = reinterpret_cast<void*>(uintptr_t(1) << 40);
  void* Bp = reinterpret_cast<void*>((uintptr_t(1) << 40) + 4096);
  void* Y = reinterpret_cast<void*>((uintptr_t(1) << 40) + 8192);
  void* W = reinterpret_cast<void*>((uintptr_t(1) << 40) + 65536);
  void* MIS = reinterpret_cast<void*>((uintptr_t(1) << 40) + 8);
  auto* a8 = static_cast<const int8_t*>(A);
  auto* b8 = static_cast<const int8_t*>(Bp);
  auto* f = static_cast<const float*>(Y);

  expect(convrot_abi_version() == CONVROT_ABI_VERSION ? 0 : 1, 0, "abi version");
  if (convrot_prepare_weight_workspace(4, 128) < 4) ++g_failed;
  if (convrot_linear_workspace(-1, 128, 4) != 0 || convrot_linear_workspace(4, 0, 4) != 0) ++g_failed;
  if (convrot_linear_workspace(100, 256, 10) < 20 * 256) ++g_failed;
  if (convrot_default_workspace(0, 4) != 0 || convrot_guarded_workspace(1, 128, 0) != 0) ++g_failed;
  g_checks += 4;

  // prepare_weight
  expect(convrot_prepare_weight(A, CONVROT_F32, 4, 128, 64, (int8_t*)Bp, (float*)Y, W, 256, nullptr),
         CONVROT_EUNSUPPORTED, "prepare: group 64");
  expect(convrot_prepare_weight(A, CONVROT_F32, 4, 200, 128, (int8_t*)Bp, (float*)Y, W, 256, nullptr),
         CONVROT_EINVAL, "prepare: K % g");
  expect(convrot_prepare_weight(A, 7, 4, 128, 128, (int8_t*)Bp, (float*)Y, W, 256, nullptr),
         CONVROT_EUNSUPPORTED, "prepare: dtype");
  expect(convrot_prepare_weight(A, CONVROT_F16, 4, 128, 128, (int8_t*)Bp, (float*)Y, W, 256, nullptr),
         CONVROT_EUNSUPPORTED, "prepare: fp16 only through _ex");
  expect(convrot_prepare_weight(nullptr, CONVROT_F32, 4, 128, 128, (int8_t*)Bp, (float*)Y, W, 256, nullptr),
         CONVROT_EINVAL, "prepare: NULL w");
  expect(convrot_prepare_weight(MIS, CONVROT_F32, 4, 128, 128, (int8_t*)Bp, (float*)Y, W, 256, nullptr),
         CONVROT_EALIGN, "prepare: misaligned w");
  expect(convrot_prepare_weight(A, CONVROT_F32, 4, 128, 128, (int8_t*)Bp, (float*)Y, W, 1, nullptr),
         CONVROT_EWORKSPACE, "prepare: workspace");
  expect(convrot_prepare_weight(A, CONVROT_F32, 0, 128, 128, (int8_t*)Bp, (float*)Y, W, 256, nullptr),
         CONVROT_EINVAL, "prepare: N = 0");
  expect(convrot_prepare_weight_ex(A, CONVROT_F16, 4, 128, 128, 5, (int8_t*)Bp, (float*)Y, W, 256, nullptr),
         CONVROT_EUNSUPPORTED, "prepare_ex: scale mode");

  // rotate + quant
  expect(convrot_rotate_quant(A, 0, 256, 128, (int8_t*)Bp, (float*)Y, nullptr), CONVROT_OK, "rotq: M = 0");
  expect(convrot_rotate_quant(A, -1, 256, 128, (int8_t*)Bp, (float*)Y, nullptr), CONVROT_EINVAL, "rotq: M < 0");
  expect(convrot_rotate_quant(A, 3, 256, 512, (int8_t*)Bp, (float*)Y, nullptr), CONVROT_EUNSUPPORTED,
         "rotq: group 512");
  expect(convrot_rotate_quant(A, 3, 131072 + 256, 256, (int8_t*)Bp, (float*)Y, nullptr), CONVROT_EINVAL,
         "rotq: K past the maximum");
  expect(convrot_rotate_quant(A, 3, 256, 128, nullptr, (float*)Y, nullptr), CONVROT_EINVAL, "rotq: NULL q");
  expect(convrot_rotate_quant(A, 3, 256, 128, (int8_t*)MIS, (float*)Y, nullptr), CONVROT_EALIGN,
         "rotq: misaligned q");
  expect(convrot_rotate_quant_ex(A, CONVROT_F32, 3, 256, 128, (int8_t*)Bp, (float*)Y, nullptr),
         CONVROT_EUNSUPPORTED, "rotq_ex: fp32 input");

  // GEMM stages
  expect(convrot_gemm_i32(a8, b8, 3, 4, 127, (int32_t*)Y, nullptr), CONVROT_EINVAL, "gemm: K = 127");
  expect(convrot_gemm_i32(a8, b8, 3, 0, 128, (int32_t*)Y, nullptr), CONVROT_EINVAL, "gemm: N = 0");
  expect(convrot_gemm_i32(a8, b8, 0, 4, 128, (int32_t*)Y, nullptr), CONVROT_OK, "gemm: M = 0");
  expect(convrot_gemm_i32(a8, b8, int64_t(1) << 31, 4, 128, (int32_t*)Y, nullptr), CONVROT_EINVAL,
         "gemm: M too large");
  expect(convrot_gemm_i32(a8, nullptr, 3, 4, 128, (int32_t*)Y, nullptr), CONVROT_EINVAL, "gemm: NULL wq");
  expect(convrot_gemm_i32(a8, b8, 3, 4, 128, (int32_t*)MIS, nullptr), CONVROT_EALIGN, "gemm: misaligned acc");
  expect(convrot_gemm_dequant(a8, f, b8, f, nullptr, Y, 3, 4, 384 + 64, nullptr), CONVROT_EINVAL,
         "dequant: K % 128");
  expect(convrot_gemm_dequant(a8, nullptr, b8, f, nullptr, Y, 3, 4, 128, nullptr), CONVROT_EINVAL,
         "dequant: NULL x_scale");
  expect(convrot_gemm_dequant_ex(a8, f, b8, f, CONVROT_SCALE_TENSOR, nullptr, Y, 9, 3, 4, 128, nullptr),
         CONVROT_EUNSUPPORTED, "dequant_ex: io dtype");

  // the whole layer
  expect(convrot_linear(A, 100, 256, b8, f, 10, 128, nullptr, Y, W, 16, nullptr), CONVROT_EWORKSPACE,
         "linear: workspace too small");
  expect(convrot_linear(A, 100, 256, b8, f, 10, 128, nullptr, Y, nullptr, 0, nullptr), CONVROT_EWORKSPACE,
         "linear: no workspace");
  expect(convrot_linear(A, 100, 256, b8, f, 10, 96, nullptr, Y, W, 1 << 20, nullptr), CONVROT_EUNSUPPORTED,
         "linear: group 96");
  expect(convrot_linear(A, 0, 256, b8, f, 10, 128, nullptr, Y, nullptr, 0, nullptr), CONVROT_OK,
         "linear: M = 0");
  expect(convrot_linear(MIS, 4, 256, b8, f, 10, 128, nullptr, Y, W, 1 << 20, nullptr), CONVROT_EALIGN,
         "linear: misaligned x");
  expect(convrot_linear_ex(A, CONVROT_F16, 4, 256, b8, f, 3, 10, 128, nullptr, Y, W, 1 << 20, nullptr),
         CONVROT_EUNSUPPORTED, "linear_ex: scale mode");

  // the no-allocation layer
  expect(convrot_linear_noalloc(A, 4, 256, b8, f, 10, 64, nullptr, Y, nullptr), CONVROT_EUNSUPPORTED,
         "noalloc: group 64");
  expect(convrot_linear_noalloc(A, 4, 200, b8, f, 10, 128, nullptr, Y, nullptr), CONVROT_EINVAL,
         "noalloc: K % g");
  expect(convrot_linear_noalloc(nullptr, 4, 256, b8, f, 10, 128, nullptr, Y, nullptr), CONVROT_EINVAL,
         "noalloc: NULL x");
  expect(convrot_linear_noalloc(A, 4, 256, b8, f, 10, 128, nullptr, MIS, nullptr), CONVROT_EALIGN,
         "noalloc: misaligned y");
  expect(convrot_linear_noalloc(A, 0, 256, b8, f, 10, 128, nullptr, Y, nullptr), CONVROT_OK, "noalloc: M = 0");

  // streamed weights
  if (convrot_stream_slot_bytes(nullptr, 0) != 0) ++g_failed;
  ++g_checks;
  expect(convrot_linear_streamed(nullptr, 0, W, 1 << 20, W, 1 << 20, nullptr, nullptr), CONVROT_OK,
         "streamed: no layers");
  expect(convrot_linear_streamed(nullptr, 2, W, 1 << 20, W, 1 << 20, nullptr, nullptr), CONVROT_EINVAL,
         "streamed: NULL layers");
  convrot_stream_layer L[2];
  std::memset(L, 0, sizeof L);
  for (auto& l : L) {
    l.x = A; l.M = 4; l.K = 256; l.N = 8; l.wq_host = b8; l.w_scale = f; l.group = 128; l.y = Y;
  }
  if (convrot_stream_slot_bytes(L, 2) < 8 * 256) ++g_failed;
  ++g_checks;
  expect(convrot_linear_streamed(L, 2, MIS, 1 << 20, W, 1 << 20, nullptr, nullptr), CONVROT_EALIGN,
         "streamed: misaligned slots");
  L[1].group = 100;
  expect(convrot_linear_streamed(L, 2, W, 1 << 20, W, 1 << 20, nullptr, nullptr), CONVROT_EUNSUPPORTED,
         "streamed: a bad layer");
  L[1].group = 128;
  expect(convrot_linear_streamed(L, 2, W, 16, W, 1 << 20, nullptr, nullptr), CONVROT_EWORKSPACE,
         "streamed: slot too small");

  // default path and guard
  expect(convrot_unpack_weight(b8, f, CONVROT_SCALE_TENSOR, 4, 200, 128, CONVROT_BF16, Y, nullptr),
         CONVROT_EINVAL, "unpack: K % g");
  expect(convrot_unpack_weight(b8, f, CONVROT_SCALE_TENSOR, 4, 256, 128, CONVROT_F32, Y, nullptr),
         CONVROT_EUNSUPPORTED, "unpack: fp32 output");
  expect(convrot_default_linear(A, CONVROT_BF16, 4, 256, b8, f, CONVROT_SCALE_TENSOR, 8, 128, nullptr, Y, W, 16,
                                nullptr),
         CONVROT_EWORKSPACE, "default: workspace");
  expect(convrot_linear_guarded(A, CONVROT_BF16, 4, 256, b8, f, CONVROT_SCALE_TENSOR, 8, 128, nullptr, Y, W, 16,
                                nullptr),
         CONVROT_EWORKSPACE, "guarded: workspace");
  expect(convrot_linear_guarded(A, CONVROT_BF16, 4, 256, nullptr, f, CONVROT_SCALE_TENSOR, 8, 128, nullptr, Y,
                                W, 1 << 30, nullptr),
         CONVROT_EINVAL, "guarded: NULL wq");
  convrot_guard_info info;
  expect(convrot_guard_query(-1, &info), CONVROT_EINVAL, "guard query: device");
  expect(convrot_guard_query(0, nullptr), CONVROT_EINVAL, "guard query: NULL");
  expect(convrot_guard_query(0, &info), CONVROT_OK, "guard query");
  expect(convrot_guard_configure(0.0, 0), CONVROT_EINVAL, "guard configure: tol 0");
  expect(convrot_guard_configure(1.0 / 0.0, 0), CONVROT_EINVAL, "guard configure: tol inf");
  expect(convrot_guard_configure(0.1, 0), CONVROT_OK, "guard configure");
  expect(convrot_guard_inject(0, 9), CONVROT_EINVAL, "guard inject: fault");
  expect(convrot_guard_inject(0, CONVROT_FAULT_MISMATCH), CONVROT_OK, "guard inject");
  expect(convrot_guard_reset(-2), CONVROT_EINVAL, "guard reset: device");
  expect(convrot_guard_reset(0), CONVROT_OK, "guard reset");

  // measurement aids
  expect(convrot_probe_mfma_i8(a8, 4096, b8, 4096, 0, 1, (int32_t*)Y, nullptr), CONVROT_EINVAL,
         "probe: blocks 0");
  expect(convrot_probe_mfma_i8(a8, 8, b8, 4096, 1, 1, (int32_t*)Y, nullptr), CONVROT_EINVAL,
         "probe: short operand");
  expect(convrot_probe_stream(A, 12, static_cast<int8_t*>(Y), nullptr), CONVROT_EINVAL,
         "stream probe: n not a multiple of 8");
  expect(convrot_probe_stream(nullptr, 8, static_cast<int8_t*>(Y), nullptr), CONVROT_EINVAL, "stream probe: NULL x");

  if (g_failed) {
    std::printf("abi_driver: %d of %d checks failed\n", g_failed, g_checks);
    return 1;
  }
  std::printf("abi_driver: %d checks passed\n", g_checks);
  return 0;
}
