// mfma_probe.hip -- measurement aids, not steps of the layer.
//
// The MFMA loop: the rate at which this GPU sustains v_mfma_i32_16x16x64_i8
// straight from registers, with no memory traffic in the loop, on operand
// bytes the caller chooses, at three waves per SIMD (the MFMA form and the
// occupancy of the GEMM's 192 x 288 tile; one wave per SIMD issuing the same
// loop, or v_mfma_i32_32x32x32_i8 at either occupancy, sustains less).
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

// 768 threads = three waves per SIMD.  Each lane takes four A and four B
// fragments (16 bytes each) from the two operand buffers and issues 16
// independent MFMAs per iteration, one per (A, B) pair, into 16 accumulators.
__global__ __launch_bounds__(768) void mfma_loop_kernel(const int8_t* __restrict__ a,
                                                        int64_t a_chunks,
                                                        const int8_t* __restrict__ b,
                                                        int64_t b_chunks, int iters,
                                                        int32_t* __restrict__ out) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 768 + threadIdx.x;
  v4i fa[4], fb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fa[i] = *reinterpret_cast<const v4i*>(a + ((t * 4 + i) % a_chunks) * 16);
    fb[i] = *reinterpret_cast<const v4i*>(b + ((t * 4 + i) % b_chunks) * 16);
  }
  v4i acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = v4i{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i & 3], fb[i >> 2], acc[i], 0, 0, 0);
  }
  int32_t s = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) s += acc[i][e];
  out[t] = s;
}

// The plain stream: the HBM traffic of rotate + quant (16-bit values in,
// one byte per value out) with no arithmetic: each thread step loads eight
// values (16 bytes) and stores their high bytes (8 bytes), grid-stride over
// the buffer.  What it sustains is the practical bandwidth ceiling for that
// traffic on this machine.
__global__ __launch_bounds__(256) void stream_probe_kernel(const uint4* __restrict__ x, int64_t n8,
                                                           uint2* __restrict__ q) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n8;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const uint4 w = x[i];
    q[i] = make_uint2(__builtin_amdgcn_perm(w.y, w.x, 0x07050301u), __builtin_amdgcn_perm(w.w, w.z, 0x07050301u));
  }
}

}  // namespace

hipError_t launch_stream_probe(const uint16_t* x, int64_t n, int8_t* q, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t n8 = n / 8;
  const int64_t blocks = (n8 + 255) / 256 < 2048 ? (n8 + 255) / 256 : 2048;
  hipLaunchKernelGGL(stream_probe_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(x), n8, reinterpret_cast<uint2*>(q));
  return hipGetLastError();
}

hipError_t launch_mfma_probe(const int8_t* a, int64_t a_bytes, const int8_t* b, int64_t b_bytes,
                             int blocks, int iters, int32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(768), 0, stream, a, a_bytes / 16, b,
                     b_bytes / 16, iters, out);
  return hipGetLastError();
}

}  // namespace convrot
