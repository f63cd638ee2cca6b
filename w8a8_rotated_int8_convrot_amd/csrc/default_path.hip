// default_path.hip -- the check of the guarded layer against the default
// (dequantizing) path.
//
// Page "int8 Compute" (InvokeAI docs), "When something goes wrong": a new
// combination of layer shape and batch-size bucket is verified once, its
// output set against the default path's; "Memory": the verification holds
// 256 output rows of each path.  The rows are spread evenly over the batch
// (row_i = i * (M - 1) / (R - 1), R = min(M, 256)); the default path runs on
// a gathered copy of those activation rows, and the comparison reduces, per
// row, the squared difference and the squared reference in fp64 with a fixed
// order, so the check gives the same verdict on every run.  Positions where
// both paths give the same infinity are agreement and are left out of both
// sums; any other non-finite value on either path counts as a mismatch.
#include "convrot_internal.hpp"

namespace convrot {
namespace {

constexpr int kThreads = 256;

// xs[i][:] = x[row_i][:], 16 bytes per lane.
__global__ __launch_bounds__(kThreads) void gather_rows_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                               int64_t K, int R, uint16_t* __restrict__ xs) {
  const int i = blockIdx.x;
  const uint4* src = reinterpret_cast<const uint4*>(x + sample_row(i, R, M) * K);
  uint4* dst = reinterpret_cast<uint4*>(xs + static_cast<int64_t>(i) * K);
  for (int64_t c = threadIdx.x; c < K / 8; c += kThreads) dst[c] = src[c];
}

template <bool F16>
__device__ inline float io_value(uint16_t b) {
  if constexpr (F16) return static_cast<float>(__builtin_bit_cast(_Float16, b));
  else return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Fixed-order workgroup sum: lane tree inside each wave, then the four wave
// sums in wave order.
__device__ inline double block_sum(double a, double* part) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) a += __shfl_xor(a, o);
  const int wave = threadIdx.x / 64;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) part[wave] = a;
  __syncthreads();
  double r = part[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) r += part[w];
  return r;
}

template <bool F16>
__global__ __launch_bounds__(kThreads) void compare_rows_kernel(
    const uint16_t* __restrict__ y, const uint16_t* __restrict__ ydef, int64_t M, int64_t N, int R,
    int flip, double* __restrict__ partial) {
  __shared__ double part[kThreads / 64];
  const int i = blockIdx.x;
  const uint16_t* a_row = y + sample_row(i, R, M) * N;
  const uint16_t* b_row = ydef + static_cast<int64_t>(i) * N;
  double d2 = 0.0, r2 = 0.0, bad = 0.0;
  for (int64_t n = threadIdx.x; n < N; n += kThreads) {
    float a = io_value<F16>(a_row[n]);
    const float b = io_value<F16>(b_row[n]);
    if (flip) a = -a;
    const bool fa = __builtin_isfinite(a), fb = __builtin_isfinite(b);
    if (!fa || !fb) {
      // the same infinity on both paths (an output beyond the io type's
      // range, e.g. fp16 past 65504) is agreement and stays out of the sums;
      // anything else that is not finite on either path is a mismatch
      const bool same_inf = !fa && !fb && a == b;
      if (!same_inf) bad += 1.0;
      continue;
    }
    const double d = static_cast<double>(a) - static_cast<double>(b);
    d2 += d * d;
    r2 += static_cast<double>(b) * static_cast<double>(b);
  }
  d2 = block_sum(d2, part);
  r2 = block_sum(r2, part);
  bad = block_sum(bad, part);
  if (threadIdx.x == 0) {
    partial[3 * i] = d2;
    partial[3 * i + 1] = r2;
    partial[3 * i + 2] = bad;
  }
}

}  // namespace

hipError_t launch_gather_rows(const uint16_t* x, int64_t M, int64_t K, int R, uint16_t* xs,
                              hipStream_t stream) {
  hipLaunchKernelGGL(gather_rows_kernel, dim3(R), dim3(kThreads), 0, stream, x, M, K, R, xs);
  return hipGetLastError();
}

hipError_t launch_compare_rows(const uint16_t* y, const uint16_t* ydef, bool f16, int64_t M, int64_t N,
                               int R, bool flip, double* partial, hipStream_t stream) {
  if (f16)
    hipLaunchKernelGGL(compare_rows_kernel<true>, dim3(R), dim3(kThreads), 0, stream, y, ydef, M, N, R,
                       flip ? 1 : 0, partial);
  else
    hipLaunchKernelGGL(compare_rows_kernel<false>, dim3(R), dim3(kThreads), 0, stream, y, ydef, M, N, R,
                       flip ? 1 : 0, partial);
  return hipGetLastError();
}

}  // namespace convrot
