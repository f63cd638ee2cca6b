// mfma_probe.hip -- a measurement aid, not a step of the layer: the rate at
// which this GPU sustains v_mfma_i32_32x32x32_i8 straight from registers, with
// no memory traffic in the loop, on operand bytes the caller chooses.
//
// Under the board's power limit the shader clock, and with it this rate,
// depends on how many operand bits toggle from one MFMA to the next: constant
// operands run near the datasheet clock, random int8 codes well below it.
// Fed with the layer's own quantized codes, the loop gives the ceiling that
// the GEMM's matrix-core rate can be compared with on the same machine and
// the same data.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "convrot_internal.hpp"

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// 256 threads = one wave per SIMD.  Each lane takes four A and four B
// fragments (16 bytes each) from the two operand buffers and issues 16
// independent MFMAs per iteration, one per (A, B) pair, into 16 accumulators.
__global__ __launch_bounds__(256) void mfma_loop_kernel(const int8_t* __restrict__ a,
                                                        int64_t a_chunks,
                                                        const int8_t* __restrict__ b,
                                                        int64_t b_chunks, int iters,
                                                        int32_t* __restrict__ out) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  v4i fa[4], fb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fa[i] = *reinterpret_cast<const v4i*>(a + ((t * 4 + i) % a_chunks) * 16);
    fb[i] = *reinterpret_cast<const v4i*>(b + ((t * 4 + i) % b_chunks) * 16);
  }
  v16i acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = v16i{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i & 3], fb[i >> 2], acc[i], 0, 0, 0);
  }
  int32_t s = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[i][e];
  out[t] = s;
}

}  // namespace

hipError_t launch_mfma_probe(const int8_t* a, int64_t a_bytes, const int8_t* b, int64_t b_bytes,
                             int blocks, int iters, int32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, stream, a, a_bytes / 16, b,
                     b_bytes / 16, iters, out);
  return hipGetLastError();
}

}  // namespace convrot
