// convrot_api.hip -- the C ABI declared in include/convrot.h: argument checks,
// workspace carving, M-slicing and kernel dispatch.  No entry point allocates
// device memory or falls back to another path on its own; only the guarded
// layer switches to the default path, by the rules stated in the header, and
// only its checking calls synchronise (with their stream).
#include "../../include/convrot.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <set>
#include <string>
#include <tuple>
#include <vector>

#include "convrot_internal.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return CONVROT_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(CONVROT_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Checks shared by the entry points that take a K dimension of codes.
int check_k(int64_t K, const char* who) {
  if (K < 128 || K > convrot::kMaxK || K % 128 != 0)
    return fail(CONVROT_EINVAL, "%s: K=%lld must be a multiple of 128 in [128, %lld]", who,
                static_cast<long long>(K), static_cast<long long>(convrot::kMaxK));
  return CONVROT_OK;
}

int check_group(int group, int64_t K, const char* who) {
  if (group != 128 && group != 256)
    return fail(CONVROT_EUNSUPPORTED, "%s: group %d is not supported (128 or 256)", who, group);
  if (K < group || K % group != 0 || K > convrot::kMaxK)
    return fail(CONVROT_EINVAL, "%s: K=%lld must be a positive multiple of the group %d, at most %lld",
                who, static_cast<long long>(K), group, static_cast<long long>(convrot::kMaxK));
  return CONVROT_OK;
}

// Rows and columns are passed to kernels as int; keep every product in range.
int check_mn(int64_t M, int64_t N, const char* who) {
  if (M < 0 || N < 1 || M > (int64_t(1) << 30) || N > (int64_t(1) << 30))
    return fail(CONVROT_EINVAL, "%s: M=%lld N=%lld out of range (0 <= M, 1 <= N, both <= 2^30)", who,
                static_cast<long long>(M), static_cast<long long>(N));
  return CONVROT_OK;
}

// Slice height of convrot_linear for a given workspace.
int64_t slice_rows(int64_t M, int64_t K, int64_t N, size_t ws_bytes) {
  const int64_t cap = M < 2 * N ? M : 2 * N;
  // codes [S, K] rounded to 256 bytes, then S floats
  int64_t fit = static_cast<int64_t>(ws_bytes / static_cast<size_t>(K + 4));
  while (fit > 0 && round_up(static_cast<size_t>(fit) * K, 256) + static_cast<size_t>(fit) * 4 > ws_bytes) --fit;
  if (fit >= cap) return cap;
  fit -= fit % 16;
  return fit;
}

}  // namespace

extern "C" {

int convrot_abi_version(void) { return CONVROT_ABI_VERSION; }

const char* convrot_last_error(void) { return g_last_error; }

size_t convrot_prepare_weight_workspace(int64_t, int64_t) { return 256; }

}  // extern "C"

namespace {

int check_io(int io_dtype, const char* who) {
  if (io_dtype != CONVROT_BF16 && io_dtype != CONVROT_F16)
    return fail(CONVROT_EUNSUPPORTED, "%s: activation/bias/output dtype %d (CONVROT_BF16 or CONVROT_F16)",
                who, io_dtype);
  return CONVROT_OK;
}

int check_scale_mode(int scale_mode, const char* who) {
  if (scale_mode != CONVROT_SCALE_TENSOR && scale_mode != CONVROT_SCALE_ROW)
    return fail(CONVROT_EUNSUPPORTED, "%s: weight scale mode %d (CONVROT_SCALE_TENSOR or CONVROT_SCALE_ROW)",
                who, scale_mode);
  return CONVROT_OK;
}

int prepare_weight_impl(const char* who, const void* w, int w_dtype, int64_t N, int64_t K, int group,
                        int scale_mode, int8_t* wq_out, float* w_scale_out, void* workspace,
                        size_t ws_bytes, void* stream) {
  if (int rc = check_group(group, K, who)) return rc;
  if (int rc = check_scale_mode(scale_mode, who)) return rc;
  if (N < 1 || N > (int64_t(1) << 31) - 1)
    return fail(CONVROT_EINVAL, "%s: N=%lld must be in [1, 2^31)", who, static_cast<long long>(N));
  if (w_dtype != CONVROT_F32 && w_dtype != CONVROT_BF16 && w_dtype != CONVROT_F16)
    return fail(CONVROT_EUNSUPPORTED, "%s: weight dtype %d (CONVROT_F32, CONVROT_BF16 or CONVROT_F16)",
                who, w_dtype);
  if (!w || !wq_out || !w_scale_out) return fail(CONVROT_EINVAL, "%s: NULL pointer", who);
  if (!aligned16(w) || !aligned16(wq_out) || (workspace && !aligned16(workspace)))
    return fail(CONVROT_EALIGN, "%s: w, wq_out and workspace must be 16-byte aligned", who);
  if (!workspace || ws_bytes < convrot_prepare_weight_workspace(N, K))
    return fail(CONVROT_EWORKSPACE, "%s: workspace of %zu bytes needed", who,
                convrot_prepare_weight_workspace(N, K));
  const int in = w_dtype == CONVROT_BF16 ? convrot::kInBf16
               : w_dtype == CONVROT_F16  ? convrot::kInF16 : convrot::kInF32;
  hipError_t e = convrot::launch_prepare_weight(w, in, scale_mode == CONVROT_SCALE_ROW, N, K, group,
                                                wq_out, w_scale_out, static_cast<uint32_t*>(workspace),
                                                static_cast<hipStream_t>(stream));
  return hip_status(e, who);
}

hipError_t rotate_quant_any(const void* x, int io_dtype, int64_t M, int64_t K, int group, int8_t* xq,
                            float* x_scale, hipStream_t stream) {
  const auto* xb = static_cast<const uint16_t*>(x);
  return io_dtype == CONVROT_F16 ? convrot::launch_rotate_quant_f16(xb, M, K, group, xq, x_scale, stream)
                                 : convrot::launch_rotate_quant(xb, M, K, group, xq, x_scale, stream);
}

int rotate_quant_impl(const char* who, const void* x, int io_dtype, int64_t M, int64_t K, int group,
                      int8_t* xq, float* x_scale, void* stream) {
  if (int rc = check_group(group, K, who)) return rc;
  if (int rc = check_io(io_dtype, who)) return rc;
  if (M < 0 || M > (int64_t(1) << 31) - 1)
    return fail(CONVROT_EINVAL, "%s: M=%lld must be in [0, 2^31)", who, static_cast<long long>(M));
  if (M == 0) return ok();
  if (!x || !xq || !x_scale) return fail(CONVROT_EINVAL, "%s: NULL pointer", who);
  if (!aligned16(x) || !aligned16(xq))
    return fail(CONVROT_EALIGN, "%s: x and xq must be 16-byte aligned", who);
  return hip_status(rotate_quant_any(x, io_dtype, M, K, group, xq, x_scale,
                                     static_cast<hipStream_t>(stream)), who);
}

int gemm_dequant_impl(const char* who, const int8_t* xq, const float* x_scale, const int8_t* wq,
                      const float* w_scale, int scale_mode, const void* bias, void* y, int io_dtype,
                      int64_t M, int64_t N, int64_t K, void* stream) {
  if (int rc = check_k(K, who)) return rc;
  if (int rc = check_mn(M, N, who)) return rc;
  if (int rc = check_io(io_dtype, who)) return rc;
  if (int rc = check_scale_mode(scale_mode, who)) return rc;
  if (M == 0) return ok();
  if (!xq || !x_scale || !wq || !w_scale || !y) return fail(CONVROT_EINVAL, "%s: NULL pointer", who);
  if (!aligned16(xq) || !aligned16(wq) || !aligned16(y))
    return fail(CONVROT_EALIGN, "%s: xq, wq and y must be 16-byte aligned", who);
  hipError_t e = convrot::launch_gemm_dequant_ex(xq, x_scale, wq, w_scale, scale_mode == CONVROT_SCALE_ROW,
                                                 static_cast<const uint16_t*>(bias),
                                                 static_cast<uint16_t*>(y), io_dtype == CONVROT_F16, M, N,
                                                 K, static_cast<hipStream_t>(stream));
  return hip_status(e, who);
}

int linear_impl(const char* who, const void* x_in, int io_dtype, int64_t M, int64_t K, const int8_t* wq,
                const float* w_scale, int scale_mode, int64_t N, int group, const void* bias_in,
                void* y_out, void* workspace, size_t ws_bytes, void* stream) {
  if (int rc = check_group(group, K, who)) return rc;
  if (int rc = check_mn(M, N, who)) return rc;
  if (int rc = check_io(io_dtype, who)) return rc;
  if (int rc = check_scale_mode(scale_mode, who)) return rc;
  if (M == 0) return ok();
  if (!x_in || !wq || !w_scale || !y_out) return fail(CONVROT_EINVAL, "%s: NULL pointer", who);
  if (!aligned16(x_in) || !aligned16(wq) || !aligned16(y_out) || (workspace && !aligned16(workspace)))
    return fail(CONVROT_EALIGN, "%s: x, wq, y and workspace must be 16-byte aligned", who);
  const int64_t S = workspace ? slice_rows(M, K, N, ws_bytes) : 0;
  // one slice of 16 rows, or of the whole slice height min(M, 2N) if that is less
  const int64_t need = std::min<int64_t>(std::min<int64_t>(M, 2 * N), 16);
  if (S < need)
    return fail(CONVROT_EWORKSPACE, "%s: workspace of %zu bytes holds %lld rows; at least %lld needed "
                "(convrot_linear_workspace gives %zu)", who, ws_bytes, static_cast<long long>(S),
                static_cast<long long>(need), convrot_linear_workspace(M, K, N));
  auto* xq = static_cast<int8_t*>(workspace);
  auto* xs = reinterpret_cast<float*>(static_cast<char*>(workspace) + round_up(static_cast<size_t>(S) * K, 256));
  const auto* x = static_cast<const uint16_t*>(x_in);
  auto* y = static_cast<uint16_t*>(y_out);
  const auto* bias = static_cast<const uint16_t*>(bias_in);
  const bool row = scale_mode == CONVROT_SCALE_ROW, f16 = io_dtype == CONVROT_F16;
  auto s = static_cast<hipStream_t>(stream);
  for (int64_t r0 = 0; r0 < M; r0 += S) {
    const int64_t rows = (M - r0) < S ? (M - r0) : S;
    hipError_t e = rotate_quant_any(x + r0 * K, io_dtype, rows, K, group, xq, xs, s);
    if (e != hipSuccess) return hip_status(e, who);
    e = convrot::launch_gemm_dequant_ex(xq, xs, wq, w_scale, row, bias, y + r0 * N, f16, rows, N, K, s);
    if (e != hipSuccess) return hip_status(e, who);
  }
  return ok();
}

}  // namespace

extern "C" {

int convrot_prepare_weight(const void* w, int w_dtype, int64_t N, int64_t K, int group,
                           int8_t* wq_out, float* w_scale_out, void* workspace, size_t ws_bytes,
                           void* stream) {
  if (w_dtype == CONVROT_F16)
    return fail(CONVROT_EUNSUPPORTED, "convrot_prepare_weight: weight dtype %d (CONVROT_F32 or "
                "CONVROT_BF16; fp16 weights through convrot_prepare_weight_ex)", w_dtype);
  return prepare_weight_impl("convrot_prepare_weight", w, w_dtype, N, K, group, CONVROT_SCALE_TENSOR,
                             wq_out, w_scale_out, workspace, ws_bytes, stream);
}

int convrot_prepare_weight_ex(const void* w, int w_dtype, int64_t N, int64_t K, int group,
                              int scale_mode, int8_t* wq_out, float* w_scale_out, void* workspace,
                              size_t ws_bytes, void* stream) {
  return prepare_weight_impl("convrot_prepare_weight_ex", w, w_dtype, N, K, group, scale_mode, wq_out,
                             w_scale_out, workspace, ws_bytes, stream);
}

size_t convrot_linear_workspace(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || K < 1 || N < 1) return 0;
  const int64_t S = M < 2 * N ? M : 2 * N;
  return round_up(static_cast<size_t>(S) * static_cast<size_t>(K), 256) + static_cast<size_t>(S) * 4;
}

}  // extern "C"

// Device memory of convrot_linear_noalloc: the codes and scales of one slice.
// In host code `scratch` names a host-side stand-in; its device address on
// each GPU is looked up once (with that GPU current) and kept per device.
static __device__ __align__(256) unsigned char scratch[CONVROT_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;

int scratch_of_current_device(const char* who, void** out) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return hip_status(e, who);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess)
      return hip_status(e, who);
    if (p == nullptr || !aligned16(p))
      return fail(CONVROT_EHIP, "%s: scratch array of device %d at an unusable address", who, dev);
    it = g_scratch_ptr.emplace(dev, p).first;
  }
  *out = it->second;
  return CONVROT_OK;
}

}  // namespace

extern "C" {

int convrot_linear_noalloc(const void* x_bf16, int64_t M, int64_t K, const int8_t* wq,
                           const float* w_scale, int64_t N, int group, const void* bias_bf16,
                           void* y_bf16, void* stream) {
  const char* who = "convrot_linear_noalloc";
  // argument errors first, before any HIP call
  if (int rc = check_group(group, K, who)) return rc;
  if (int rc = check_mn(M, N, who)) return rc;
  if (M == 0) return ok();
  if (!x_bf16 || !wq || !w_scale || !y_bf16) return fail(CONVROT_EINVAL, "%s: NULL pointer", who);
  if (!aligned16(x_bf16) || !aligned16(wq) || !aligned16(y_bf16))
    return fail(CONVROT_EALIGN, "%s: x, wq and y must be 16-byte aligned", who);
  const size_t cap = CONVROT_NOALLOC_SCRATCH_BYTES;
  const int64_t need = std::min<int64_t>(std::min<int64_t>(M, 2 * N), 16);
  if (slice_rows(M, K, N, cap) < need)
    return fail(CONVROT_EWORKSPACE, "%s: a slice of %lld tokens of K=%lld does not fit the %zu-byte scratch array",
                who, static_cast<long long>(need), static_cast<long long>(K), cap);
  void* ws = nullptr;
  if (int rc = scratch_of_current_device(who, &ws)) return rc;
  return linear_impl(who, x_bf16, CONVROT_BF16, M, K, wq, w_scale, CONVROT_SCALE_TENSOR, N, group, bias_bf16,
                     y_bf16, ws, cap, stream);
}

int convrot_rotate_quant(const void* x_bf16, int64_t M, int64_t K, int group, int8_t* xq,
                         float* x_scale, void* stream) {
  return rotate_quant_impl("convrot_rotate_quant", x_bf16, CONVROT_BF16, M, K, group, xq, x_scale,
                           stream);
}

int convrot_rotate_quant_ex(const void* x, int x_dtype, int64_t M, int64_t K, int group, int8_t* xq,
                            float* x_scale, void* stream) {
  return rotate_quant_impl("convrot_rotate_quant_ex", x, x_dtype, M, K, group, xq, x_scale, stream);
}

int convrot_gemm_i32(const int8_t* xq, const int8_t* wq, int64_t M, int64_t N, int64_t K,
                     int32_t* acc, void* stream) {
  const char* who = "convrot_gemm_i32";
  if (int rc = check_k(K, who)) return rc;
  if (int rc = check_mn(M, N, who)) return rc;
  if (M == 0) return ok();
  if (!xq || !wq || !acc) return fail(CONVROT_EINVAL, "%s: NULL pointer", who);
  if (!aligned16(xq) || !aligned16(wq) || !aligned16(acc))
    return fail(CONVROT_EALIGN, "%s: xq, wq and acc must be 16-byte aligned", who);
  hipError_t e = convrot::launch_gemm_i32(xq, wq, acc, M, N, K, static_cast<hipStream_t>(stream));
  return hip_status(e, who);
}

int convrot_gemm_dequant(const int8_t* xq, const float* x_scale, const int8_t* wq,
                         const float* w_scale, const void* bias_bf16, void* y_bf16, int64_t M,
                         int64_t N, int64_t K, void* stream) {
  return gemm_dequant_impl("convrot_gemm_dequant", xq, x_scale, wq, w_scale, CONVROT_SCALE_TENSOR,
                           bias_bf16, y_bf16, CONVROT_BF16, M, N, K, stream);
}

int convrot_gemm_dequant_ex(const int8_t* xq, const float* x_scale, const int8_t* wq,
                            const float* w_scale, int scale_mode, const void* bias, void* y,
                            int io_dtype, int64_t M, int64_t N, int64_t K, void* stream) {
  return gemm_dequant_impl("convrot_gemm_dequant_ex", xq, x_scale, wq, w_scale, scale_mode, bias, y,
                           io_dtype, M, N, K, stream);
}

int convrot_linear(const void* x_bf16, int64_t M, int64_t K, const int8_t* wq, const float* w_scale,
                   int64_t N, int group, const void* bias_bf16, void* y_bf16, void* workspace,
                   size_t ws_bytes, void* stream) {
  return linear_impl("convrot_linear", x_bf16, CONVROT_BF16, M, K, wq, w_scale, CONVROT_SCALE_TENSOR, N,
                     group, bias_bf16, y_bf16, workspace, ws_bytes, stream);
}

int convrot_linear_ex(const void* x, int io_dtype, int64_t M, int64_t K, const int8_t* wq,
                      const float* w_scale, int scale_mode, int64_t N, int group, const void* bias,
                      void* y, void* workspace, size_t ws_bytes, void* stream) {
  return linear_impl("convrot_linear_ex", x, io_dtype, M, K, wq, w_scale, scale_mode, N, group, bias, y,
                     workspace, ws_bytes, stream);
}

size_t convrot_stream_slot_bytes(const convrot_stream_layer* layers, int n_layers) {
  if (!layers || n_layers < 1) return 0;
  size_t mx = 0;
  for (int i = 0; i < n_layers; ++i) {
    const convrot_stream_layer& L = layers[i];
    if (L.N > 0 && L.K > 0) {
      const size_t b = static_cast<size_t>(L.N) * static_cast<size_t>(L.K);
      if (b > mx) mx = b;
    }
  }
  return round_up(mx, 256);
}

int convrot_linear_streamed(const convrot_stream_layer* layers, int n_layers, void* slots,
                            size_t slot_bytes, void* workspace, size_t ws_bytes, void* copy_stream,
                            void* stream) {
  const char* who = "convrot_linear_streamed";
  if (n_layers < 0 || (n_layers > 0 && !layers))
    return fail(CONVROT_EINVAL, "%s: n_layers=%d with %s layers", who, n_layers, layers ? "non-NULL" : "NULL");
  if (n_layers == 0) return ok();
  if (!slots || !aligned16(slots) || slot_bytes % 16 != 0)
    return fail(slots ? CONVROT_EALIGN : CONVROT_EINVAL, "%s: slots must be a 16-byte aligned device buffer "
                "of 2 * slot_bytes, slot_bytes a multiple of 16", who);
  // every layer is checked before anything is queued
  for (int i = 0; i < n_layers; ++i) {
    const convrot_stream_layer& L = layers[i];
    if (int rc = check_group(L.group, L.K, who)) return rc;
    if (int rc = check_mn(L.M, L.N, who)) return rc;
    if (!L.wq_host || !L.w_scale || (L.M > 0 && (!L.x || !L.y)))
      return fail(CONVROT_EINVAL, "%s: layer %d: NULL pointer", who, i);
    if ((L.M > 0 && (!aligned16(L.x) || !aligned16(L.y))) || (workspace && !aligned16(workspace)))
      return fail(CONVROT_EALIGN, "%s: layer %d: x, y and workspace must be 16-byte aligned", who, i);
    if (static_cast<size_t>(L.N) * static_cast<size_t>(L.K) > slot_bytes)
      return fail(CONVROT_EWORKSPACE, "%s: layer %d: N*K=%lld bytes exceed slot_bytes=%zu", who, i,
                  static_cast<long long>(L.N * L.K), slot_bytes);
    const int64_t S = workspace ? slice_rows(L.M, L.K, L.N, ws_bytes) : 0;
    const int64_t need = std::min<int64_t>(std::min<int64_t>(L.M, 2 * L.N), 16);
    if (S < need)
      return fail(CONVROT_EWORKSPACE, "%s: layer %d: workspace of %zu bytes holds %lld rows; at least %lld "
                  "needed", who, i, ws_bytes, static_cast<long long>(S), static_cast<long long>(need));
  }
  for (int i = 0; i < n_layers; ++i) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, layers[i].wq_host) != hipSuccess ||
        attr.type != hipMemoryTypeHost) {
      (void)hipGetLastError();   // an unregistered pointer leaves an error behind: clear it
      return fail(CONVROT_EINVAL, "%s: layer %d: wq_host is not pinned host memory", who, i);
    }
  }

  auto cs = static_cast<hipStream_t>(copy_stream);
  auto s = static_cast<hipStream_t>(stream);
  hipEvent_t ev[5] = {};   // copied[2], computed[2], start
  for (auto& e : ev)
    if (hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming); r != hipSuccess) {
      for (auto& d : ev) if (d) (void)hipEventDestroy(d);
      return hip_status(r, who);
    }
  hipEvent_t* copied = ev;
  hipEvent_t* computed = ev + 2;
  int rc = CONVROT_OK;
  auto check = [&](hipError_t e) { if (e != hipSuccess && rc == CONVROT_OK) rc = hip_status(e, who); return e == hipSuccess; };
  // the slots may still be read by work queued earlier on `stream`
  if (check(hipEventRecord(ev[4], s)) && check(hipStreamWaitEvent(cs, ev[4], 0))) {
    for (int i = 0; i < n_layers && rc == CONVROT_OK; ++i) {
      const convrot_stream_layer& L = layers[i];
      const int k = i & 1;
      auto* slot = static_cast<int8_t*>(slots) + static_cast<size_t>(k) * slot_bytes;
      if (i >= 2 && !check(hipStreamWaitEvent(cs, computed[k], 0))) break;
      if (!check(hipMemcpyAsync(slot, L.wq_host, static_cast<size_t>(L.N) * static_cast<size_t>(L.K),
                                hipMemcpyHostToDevice, cs))) break;
      if (!check(hipEventRecord(copied[k], cs)) || !check(hipStreamWaitEvent(s, copied[k], 0))) break;
      const int r = linear_impl(who, L.x, CONVROT_BF16, L.M, L.K, slot, L.w_scale, CONVROT_SCALE_TENSOR,
                                L.N, L.group, L.bias, L.y, workspace, ws_bytes, stream);
      if (r != CONVROT_OK) { rc = r; break; }
      if (!check(hipEventRecord(computed[k], s))) break;
    }
  }
  for (auto& e : ev) (void)hipEventDestroy(e);   // released once the queued work has passed them
  return rc == CONVROT_OK ? ok() : rc;
}

// ---------------------------------------------------------------- default path and guarded layer

}  // extern "C"

namespace {

constexpr int kCheckRows = 256;

size_t default_ws(int64_t K, int64_t N) {
  return round_up(2 * static_cast<size_t>(N) * static_cast<size_t>(K), 256);
}

// Workspace of a checking call: the unpacked weight, the gathered activation
// rows, the default path's output rows and the per-row sums.
struct CheckLayout {
  int R;
  size_t xs, ydef, partial, total;
};
CheckLayout check_layout(int64_t M, int64_t K, int64_t N) {
  CheckLayout L;
  L.R = static_cast<int>(M < kCheckRows ? M : kCheckRows);
  const size_t R = static_cast<size_t>(L.R);
  L.xs = default_ws(K, N);
  L.ydef = L.xs + round_up(2 * R * static_cast<size_t>(K), 256);
  L.partial = L.ydef + round_up(2 * R * static_cast<size_t>(N), 256);
  L.total = L.partial + round_up(3 * sizeof(double) * R, 256);
  return L;
}

int unpack_impl(const char* who, const int8_t* wq, const float* w_scale, int scale_mode, int64_t N,
                int64_t K, int group, int out_dtype, void* wu, void* stream) {
  if (int rc = check_group(group, K, who)) return rc;
  if (int rc = check_scale_mode(scale_mode, who)) return rc;
  if (int rc = check_io(out_dtype, who)) return rc;
  if (N < 1 || N > (int64_t(1) << 31) - 1)
    return fail(CONVROT_EINVAL, "%s: N=%lld must be in [1, 2^31)", who, static_cast<long long>(N));
  if (!wq || !w_scale || !wu) return fail(CONVROT_EINVAL, "%s: NULL pointer", who);
  if (!aligned16(wq) || !aligned16(wu)) return fail(CONVROT_EALIGN, "%s: wq and wu must be 16-byte aligned", who);
  return hip_status(convrot::launch_unpack_weight(wq, w_scale, scale_mode == CONVROT_SCALE_ROW, N, K, group,
                                                  out_dtype == CONVROT_F16, static_cast<uint16_t*>(wu),
                                                  static_cast<hipStream_t>(stream)),
                    who);
}

// Checks shared by the default path and the guarded layer (those of
// convrot_linear_ex except the workspace).
int check_layer(const char* who, const void* x, int io_dtype, int64_t M, int64_t K, const int8_t* wq,
                const float* w_scale, int scale_mode, int64_t N, int group, void* y, void* workspace) {
  if (int rc = check_group(group, K, who)) return rc;
  if (int rc = check_mn(M, N, who)) return rc;
  if (int rc = check_io(io_dtype, who)) return rc;
  if (int rc = check_scale_mode(scale_mode, who)) return rc;
  if (M == 0) return CONVROT_OK;
  if (!x || !wq || !w_scale || !y) return fail(CONVROT_EINVAL, "%s: NULL pointer", who);
  if (!aligned16(x) || !aligned16(wq) || !aligned16(y) || (workspace && !aligned16(workspace)))
    return fail(CONVROT_EALIGN, "%s: x, wq, y and workspace must be 16-byte aligned", who);
  return CONVROT_OK;
}

int default_impl(const char* who, const void* x, int io_dtype, int64_t M, int64_t K, const int8_t* wq,
                 const float* w_scale, int scale_mode, int64_t N, int group, const void* bias, void* y,
                 void* workspace, size_t ws_bytes, void* stream) {
  if (int rc = check_layer(who, x, io_dtype, M, K, wq, w_scale, scale_mode, N, group, y, workspace)) return rc;
  if (M == 0) return ok();
  if (!workspace || ws_bytes < default_ws(K, N))
    return fail(CONVROT_EWORKSPACE, "%s: workspace of %zu bytes needed (the unpacked weight)", who,
                default_ws(K, N));
  auto s = static_cast<hipStream_t>(stream);
  const bool f16 = io_dtype == CONVROT_F16;
  auto* wu = static_cast<uint16_t*>(workspace);
  hipError_t e = convrot::launch_unpack_weight(wq, w_scale, scale_mode == CONVROT_SCALE_ROW, N, K, group, f16,
                                               wu, s);
  if (e != hipSuccess) return hip_status(e, who);
  e = convrot::launch_gemm_default(static_cast<const uint16_t*>(x), wu, static_cast<const uint16_t*>(bias),
                                   static_cast<uint16_t*>(y), f16, M, N, K, s);
  return hip_status(e, who);
}

// ---- guard state, per device
struct GuardKey {
  int64_t N, K;
  int group, io, mode;
  int64_t bucket;
  bool operator<(const GuardKey& o) const {
    return std::tie(N, K, group, io, mode, bucket) < std::tie(o.N, o.K, o.group, o.io, o.mode, o.bucket);
  }
};

struct GuardState {
  bool fallback = false;
  bool announced = false;
  std::set<GuardKey> checked;
  int64_t checks_run = 0;
  double last_error = -1.0;
  int inject = CONVROT_FAULT_NONE;
  std::string message;
};

std::mutex g_guard_mu;
std::map<int, GuardState> g_guard;
double g_guard_tol = 0.1;
bool g_guard_log = true;

// Called with g_guard_mu held.
void guard_log(GuardState& st, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  st.message = buf;
  if (g_guard_log) fprintf(stderr, "%s\n", buf);
}

void guard_fall_back(int dev, const char* why) {
  std::lock_guard<std::mutex> lock(g_guard_mu);
  GuardState& st = g_guard[dev];
  if (!st.fallback) {
    st.fallback = true;
    guard_log(st, "convrot: %s on device %d; this device uses the default path until the process ends", why,
              dev);
  }
}

int64_t token_bucket(int64_t M) {
  int64_t b = 1;
  while (b < M) b <<= 1;
  return b;
}

}  // namespace

extern "C" {

size_t convrot_default_workspace(int64_t K, int64_t N) {
  if (K < 1 || N < 1) return 0;
  return default_ws(K, N);
}

int convrot_unpack_weight(const int8_t* wq, const float* w_scale, int scale_mode, int64_t N, int64_t K,
                          int group, int out_dtype, void* wu, void* stream) {
  return unpack_impl("convrot_unpack_weight", wq, w_scale, scale_mode, N, K, group, out_dtype, wu, stream);
}

int convrot_default_linear(const void* x, int io_dtype, int64_t M, int64_t K, const int8_t* wq,
                           const float* w_scale, int scale_mode, int64_t N, int group, const void* bias,
                           void* y, void* workspace, size_t ws_bytes, void* stream) {
  return default_impl("convrot_default_linear", x, io_dtype, M, K, wq, w_scale, scale_mode, N, group, bias, y,
                      workspace, ws_bytes, stream);
}

size_t convrot_guarded_workspace(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || K < 1 || N < 1) return 0;
  const size_t a = convrot_linear_workspace(M, K, N);
  const size_t b = check_layout(M, K, N).total;
  return a > b ? a : b;
}

int convrot_linear_guarded(const void* x, int io_dtype, int64_t M, int64_t K, const int8_t* wq,
                           const float* w_scale, int scale_mode, int64_t N, int group, const void* bias,
                           void* y, void* workspace, size_t ws_bytes, void* stream) {
  const char* who = "convrot_linear_guarded";
  if (int rc = check_layer(who, x, io_dtype, M, K, wq, w_scale, scale_mode, N, group, y, workspace)) return rc;
  if (M == 0) return ok();
  if (!workspace || ws_bytes < convrot_guarded_workspace(M, K, N))
    return fail(CONVROT_EWORKSPACE, "%s: workspace of %zu bytes needed (convrot_guarded_workspace)", who,
                convrot_guarded_workspace(M, K, N));
  auto s = static_cast<hipStream_t>(stream);
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return hip_status(e, who);
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipError_t e = hipStreamIsCapturing(s, &capture); e != hipSuccess) return hip_status(e, who);
  const GuardKey key{N, K, group, io_dtype, scale_mode, token_bucket(M)};

  bool fallback = false, need_check = false;
  int inject = CONVROT_FAULT_NONE;
  {
    std::lock_guard<std::mutex> lock(g_guard_mu);
    GuardState& st = g_guard[dev];
    fallback = st.fallback;
    if (!fallback) {
      need_check = st.checked.count(key) == 0 || st.inject == CONVROT_FAULT_MISMATCH;
      if (need_check && capture != hipStreamCaptureStatusNone)
        return fail(CONVROT_EUNSUPPORTED, "%s: the first call for this layer shape and token bucket checks its "
                    "result and cannot be captured; run it once before capturing", who);
      inject = st.inject;
      st.inject = CONVROT_FAULT_NONE;
      if (!st.announced) {
        st.announced = true;
        guard_log(st, "convrot: rotated int8 layers on device %d run on the int8 matrix cores", dev);
      }
    }
  }
  if (fallback)
    return default_impl(who, x, io_dtype, M, K, wq, w_scale, scale_mode, N, group, bias, y, workspace,
                        ws_bytes, stream);

  int rc = inject == CONVROT_FAULT_KERNEL
               ? fail(CONVROT_EHIP, "%s: injected kernel failure", who)
               : linear_impl(who, x, io_dtype, M, K, wq, w_scale, scale_mode, N, group, bias, y, workspace,
                             ws_bytes, stream);
  if (rc == CONVROT_EHIP) {
    std::string why = std::string("the int8 layer failed (") + g_last_error + ")";
    guard_fall_back(dev, why.c_str());
    return default_impl(who, x, io_dtype, M, K, wq, w_scale, scale_mode, N, group, bias, y, workspace,
                        ws_bytes, stream);
  }
  if (rc != CONVROT_OK || !need_check) return rc;

  // the check: the default path on R rows spread over the batch
  const CheckLayout L = check_layout(M, K, N);
  char* ws = static_cast<char*>(workspace);
  auto* wu = reinterpret_cast<uint16_t*>(ws);
  auto* xs = reinterpret_cast<uint16_t*>(ws + L.xs);
  auto* ydef = reinterpret_cast<uint16_t*>(ws + L.ydef);
  auto* partial = reinterpret_cast<double*>(ws + L.partial);
  const bool f16 = io_dtype == CONVROT_F16;
  hipError_t e = convrot::launch_unpack_weight(wq, w_scale, scale_mode == CONVROT_SCALE_ROW, N, K, group, f16,
                                               wu, s);
  if (e == hipSuccess) e = convrot::launch_gather_rows(static_cast<const uint16_t*>(x), M, K, L.R, xs, s);
  if (e == hipSuccess)
    e = convrot::launch_gemm_default(xs, wu, static_cast<const uint16_t*>(bias), ydef, f16, L.R, N, K, s);
  if (e == hipSuccess)
    e = convrot::launch_compare_rows(static_cast<const uint16_t*>(y), ydef, f16, M, N, L.R,
                                     inject == CONVROT_FAULT_MISMATCH, partial, s);
  std::vector<double> host(3 * static_cast<size_t>(L.R));
  if (e == hipSuccess)
    e = hipMemcpyAsync(host.data(), partial, host.size() * sizeof(double), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, who);
  double d2 = 0.0, r2 = 0.0, bad = 0.0;
  for (int i = 0; i < L.R; ++i) {
    d2 += host[3 * i];
    r2 += host[3 * i + 1];
    bad += host[3 * i + 2];
  }
  const double rel = r2 > 0.0 ? std::sqrt(d2 / r2) : std::sqrt(d2);
  bool match;
  {
    std::lock_guard<std::mutex> lock(g_guard_mu);
    GuardState& st = g_guard[dev];
    match = bad == 0.0 && rel <= g_guard_tol;
    st.checks_run += 1;
    st.last_error = rel;
    if (match) st.checked.insert(key);
  }
  if (match) return ok();
  char why[160];
  snprintf(why, sizeof why, "the int8 result for N=%lld K=%lld, up to %lld tokens, does not match the default "
           "path (relative error %.3g, %.0f non-finite values)", static_cast<long long>(N),
           static_cast<long long>(K), static_cast<long long>(key.bucket), rel, bad);
  guard_fall_back(dev, why);
  return default_impl(who, x, io_dtype, M, K, wq, w_scale, scale_mode, N, group, bias, y, workspace, ws_bytes,
                      stream);
}

int convrot_guard_query(int device, convrot_guard_info* info) {
  if (device < 0 || !info) return fail(CONVROT_EINVAL, "convrot_guard_query: device %d, info %p", device,
                                       static_cast<void*>(info));
  std::lock_guard<std::mutex> lock(g_guard_mu);
  GuardState st;
  auto it = g_guard.find(device);
  if (it != g_guard.end()) st = it->second;
  info->fallback = st.fallback ? 1 : 0;
  info->checked = static_cast<int64_t>(st.checked.size());
  info->checks_run = st.checks_run;
  info->last_error = st.last_error;
  snprintf(info->message, sizeof info->message, "%s", st.message.c_str());
  return ok();
}

int convrot_guard_reset(int device) {
  if (device < 0) return fail(CONVROT_EINVAL, "convrot_guard_reset: device %d", device);
  std::lock_guard<std::mutex> lock(g_guard_mu);
  g_guard.erase(device);
  return ok();
}

int convrot_guard_configure(double tol, int log_to_stderr) {
  if (!(tol > 0.0) || !std::isfinite(tol))
    return fail(CONVROT_EINVAL, "convrot_guard_configure: tolerance %g must be finite and > 0", tol);
  std::lock_guard<std::mutex> lock(g_guard_mu);
  g_guard_tol = tol;
  g_guard_log = log_to_stderr != 0;
  return ok();
}

int convrot_guard_inject(int device, int fault) {
  if (device < 0 || (fault != CONVROT_FAULT_NONE && fault != CONVROT_FAULT_MISMATCH &&
                     fault != CONVROT_FAULT_KERNEL))
    return fail(CONVROT_EINVAL, "convrot_guard_inject: device %d, fault %d", device, fault);
  std::lock_guard<std::mutex> lock(g_guard_mu);
  g_guard[device].inject = fault;
  return ok();
}

// ---------------------------------------------------------------- measurement aid

int convrot_probe_mfma_i8(const int8_t* a, int64_t a_bytes, const int8_t* b, int64_t b_bytes,
                          int blocks, int iters, int32_t* out, void* stream) {
  const char* who = "convrot_probe_mfma_i8";
  if (!a || !b || !out) return fail(CONVROT_EINVAL, "%s: NULL pointer", who);
  if (a_bytes < 16 || b_bytes < 16 || blocks < 1 || blocks > (1 << 20) || iters < 1)
    return fail(CONVROT_EINVAL, "%s: operand buffers need 16+ bytes, blocks in [1, 2^20], iters >= 1",
                who);
  if (!aligned16(a) || !aligned16(b) || !aligned16(out))
    return fail(CONVROT_EALIGN, "%s: a, b and out must be 16-byte aligned", who);
  return hip_status(convrot::launch_mfma_probe(a, a_bytes, b, b_bytes, blocks, iters, out,
                                               static_cast<hipStream_t>(stream)),
                    who);
}

int convrot_probe_stream(const void* x_16, int64_t n, int8_t* q, void* stream) {
  const char* who = "convrot_probe_stream";
  if (n < 0 || n % 8 != 0) return fail(CONVROT_EINVAL, "%s: n = %lld must be a non-negative multiple of 8", who,
                                       static_cast<long long>(n));
  if (n > 0 && (!x_16 || !q)) return fail(CONVROT_EINVAL, "%s: NULL pointer", who);
  if (n > 0 && (!aligned16(x_16) || !aligned16(q)))
    return fail(CONVROT_EALIGN, "%s: x and q must be 16-byte aligned", who);
  return hip_status(convrot::launch_stream_probe(static_cast<const uint16_t*>(x_16), n, q,
                                                 static_cast<hipStream_t>(stream)),
                    who);
}

}  // extern "C"
