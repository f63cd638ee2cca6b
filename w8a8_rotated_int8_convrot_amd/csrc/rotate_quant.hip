// rotate_quant.hip -- group-wise Walsh-Hadamard rotation + int8 quantization
// for gfx950.
//
// What is computed (page "int8 Compute", InvokeAI docs, opening section: each
// layer rotates and quantizes its input to int8 per token; the weight is an
// int8_tensorwise build; rotation groups per "What stays on the default
// path"):
//   v      = x_row rotated block by block by H_g / sqrt(g)
//   scale  = max |v| / 127  (per token for activations, one for a weight)
//   code   = clamp(rne(v / scale), -127, 127), 0 where scale == 0
// The rotation is the fp32 radix-2 butterfly with half-span h = 1, 2, ...,
// g/2 ((a, b) -> (a + b, a - b)) followed by one multiply by the float nearest
// to 1/sqrt(g).  Every add happens in that order on the GPU too, so the codes
// are bit-identical to a sequential evaluation of the same butterfly.
//
// Layout on the device: one workgroup of 256 threads per row.  A thread owns
// up to CPT chunks of 8 consecutive elements (16-byte bf16 loads, 8-byte code
// stores, both coalesced across the wave); chunk c of a segment of
// 256 * 8 * CPT elements sits in thread c % 256.  Stages h = 1, 2, 4 stay inside a thread; stage h = 8 * 2^t pairs
// thread lanes whose index differs in bit t, so a g-group spans g/8
// consecutive lanes of one wavefront and the exchange is a lane shuffle.
// Rows of up to 256 * 8 * kMaxChunksPerThread elements are rotated once and
// held in registers; longer rows are rotated twice (absmax pass, then code pass),
// which gives the same values because the arithmetic is deterministic.
#include "convrot_internal.hpp"

namespace convrot {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunksPerThread = 6;   // rows up to 12288 elements are rotated once

// The float nearest to 1/sqrt(g): 2^-3.5 rounds to 0x3db504f3 for g = 128;
// 2^-4 is exact for g = 256.
template <int G> struct RotScale;
template <> struct RotScale<128> { static constexpr float value = 0x1.6a09e6p-4f; };
template <> struct RotScale<256> { static constexpr float value = 0x1p-4f; };

enum Mode { kActQuant = 0, kWeightAbsmax = 1, kWeightQuant = 2 };

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Load 8 consecutive inputs as fp32.
__device__ inline void load8(const uint16_t* p, float (&v)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
  v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
  v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}
__device__ inline void load8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Butterfly of one 8-element chunk that is part of a g-group spread over g/8
// lanes; `lane_in_group` is this lane's index inside the group.
template <int G>
__device__ inline void rotate_chunk(float (&v)[8], int lane_in_group) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int t = 1; t < G / 8; t <<= 1) {
    const bool upper = (lane_in_group & t) != 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = __shfl_xor(v[i], t);
      // lower element keeps a + b, upper element keeps a - b (a = lower)
      v[i] = upper ? (p - v[i]) : (v[i] + p);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = v[i] * RotScale<G>::value;
}

__device__ inline int quant_code(float v, float s) {
  float r = __builtin_rintf(v / s);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return static_cast<int>(r);
}

__device__ inline uint2 pack8(const float (&v)[8], float s) {
  uint32_t lo = 0, hi = 0;
  if (s != 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= (static_cast<uint32_t>(quant_code(v[i], s)) & 0xffu) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= (static_cast<uint32_t>(quant_code(v[4 + i], s)) & 0xffu) << (8 * i);
  }
  return make_uint2(lo, hi);
}

// Maximum over the workgroup (max is exact and order-free).
__device__ inline float block_max(float a) {
  __shared__ float part[kThreads / 64];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
  const int wave = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) part[wave] = a;
  __syncthreads();
  float r = part[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, part[w]);
  return r;
}

template <int G, int CPT, typename In, int MODE>
__global__ __launch_bounds__(kThreads) void rotate_rows_kernel(
    const In* __restrict__ x, int64_t K, int8_t* __restrict__ q, float* __restrict__ scale,
    uint32_t* __restrict__ amax_cell) {
  constexpr int kSegment = kThreads * 8 * CPT;
  const int64_t row = blockIdx.x;
  const In* xr = x + row * K;
  const int tid = threadIdx.x;
  const int lane_in_group = tid % (G / 8);
  const int nseg = static_cast<int>((K + kSegment - 1) / kSegment);

  // Chunk slots past the row end are skipped lane by lane.  K is a multiple
  // of G, so a g-group is either wholly inside the row or wholly outside,
  // and the lane exchange of a valid group only reads valid lanes.
  float v[CPT][8];
  float amax = 0.0f;

  // absmax pass (for one-segment rows the rotated values stay in registers)
  for (int seg = 0; seg < nseg; ++seg) {
    const int64_t base = static_cast<int64_t>(seg) * kSegment;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int64_t e = base + (static_cast<int64_t>(j) * kThreads + tid) * 8;
      if (e < K) load8(xr + e, v[j]);
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int64_t e = base + (static_cast<int64_t>(j) * kThreads + tid) * 8;
      if (e < K) {
        rotate_chunk<G>(v[j], lane_in_group);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[j][i]));
      }
    }
  }

  if (MODE == kWeightAbsmax) {
    const float m = block_max(amax);
    if (tid == 0) atomicMax(amax_cell, __float_as_uint(m));  // m >= 0: bit order = value order
    return;
  }

  float s;
  if (MODE == kActQuant) {
    s = block_max(amax) / 127.0f;
    if (tid == 0) scale[row] = s;
  } else {
    s = __uint_as_float(*amax_cell) / 127.0f;
    if (row == 0 && tid == 0) scale[0] = s;
  }

  int8_t* qr = q + row * K;
  for (int seg = 0; seg < nseg; ++seg) {
    const int64_t base = static_cast<int64_t>(seg) * kSegment;
    if (nseg > 1) {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int64_t e = base + (static_cast<int64_t>(j) * kThreads + tid) * 8;
        if (e < K) load8(xr + e, v[j]);
      }
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int64_t e = base + (static_cast<int64_t>(j) * kThreads + tid) * 8;
        if (e < K) rotate_chunk<G>(v[j], lane_in_group);
      }
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int64_t e = base + (static_cast<int64_t>(j) * kThreads + tid) * 8;
      if (e < K) *reinterpret_cast<uint2*>(qr + e) = pack8(v[j], s);
    }
  }
}

__global__ void zero_word_kernel(uint32_t* p) { *p = 0u; }

template <int G, int CPT, typename In, int MODE>
hipError_t launch_rows(const In* x, int64_t rows, int64_t K, int8_t* q, float* scale,
                       uint32_t* cell, hipStream_t stream) {
  hipLaunchKernelGGL((rotate_rows_kernel<G, CPT, In, MODE>), dim3(static_cast<uint32_t>(rows)),
                     dim3(kThreads), 0, stream, x, K, q, scale, cell);
  return hipGetLastError();
}

// Chunks per thread: the fewest that hold the row (2048 elements per chunk
// slot), else the maximum with a two-pass row.
template <int G, typename In, int MODE>
hipError_t launch_rows_k(const In* x, int64_t rows, int64_t K, int8_t* q, float* scale,
                         uint32_t* cell, hipStream_t stream) {
  const int64_t slots = (K + kThreads * 8 - 1) / (kThreads * 8);
  if (slots <= 1) return launch_rows<G, 1, In, MODE>(x, rows, K, q, scale, cell, stream);
  if (slots <= 2) return launch_rows<G, 2, In, MODE>(x, rows, K, q, scale, cell, stream);
  if (slots <= 4) return launch_rows<G, 4, In, MODE>(x, rows, K, q, scale, cell, stream);
  return launch_rows<G, kMaxChunksPerThread, In, MODE>(x, rows, K, q, scale, cell, stream);
}

template <typename In, int MODE>
hipError_t dispatch_group(int group, const In* x, int64_t rows, int64_t K, int8_t* q,
                          float* scale, uint32_t* cell, hipStream_t stream) {
  if (group == 128) return launch_rows_k<128, In, MODE>(x, rows, K, q, scale, cell, stream);
  return launch_rows_k<256, In, MODE>(x, rows, K, q, scale, cell, stream);
}

}  // namespace

hipError_t launch_rotate_quant(const uint16_t* x, int64_t M, int64_t K, int group, int8_t* q,
                               float* scale, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  return dispatch_group<uint16_t, kActQuant>(group, x, M, K, q, scale, nullptr, stream);
}

hipError_t launch_prepare_weight(const void* w, bool in_bf16, int64_t N, int64_t K, int group,
                                 int8_t* wq, float* w_scale, uint32_t* amax_cell,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(1), 0, stream, amax_cell);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (in_bf16) {
    const auto* x = static_cast<const uint16_t*>(w);
    e = dispatch_group<uint16_t, kWeightAbsmax>(group, x, N, K, nullptr, nullptr, amax_cell, stream);
    if (e != hipSuccess) return e;
    return dispatch_group<uint16_t, kWeightQuant>(group, x, N, K, wq, w_scale, amax_cell, stream);
  }
  const auto* x = static_cast<const float*>(w);
  e = dispatch_group<float, kWeightAbsmax>(group, x, N, K, nullptr, nullptr, amax_cell, stream);
  if (e != hipSuccess) return e;
  return dispatch_group<float, kWeightQuant>(group, x, N, K, wq, w_scale, amax_cell, stream);
}

}  // namespace convrot
