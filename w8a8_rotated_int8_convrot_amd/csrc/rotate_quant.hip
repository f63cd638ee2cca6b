// rotate_quant.hip -- group-wise Walsh-Hadamard rotation + int8 quantization
// for gfx950.
//
// What is computed (page "int8 Compute", InvokeAI docs, opening section: a
// layer's activation is rotated, then given int8 codes with one scale per
// token; its weight holds int8 codes with a single tensor scale; the rotation
// works in groups, "What stays on the default path"):
//   v      = x_row rotated block by block by H_g / sqrt(g)
//   scale  = max |v| / 127  (per token for activations, one for a weight)
//   code   = clamp(rne(v / scale), -127, 127), 0 where scale == 0
// The rotation is the fp32 radix-2 butterfly with half-span h = 1, 2, ...,
// g/2 ((a, b) -> (a + b, a - b)) followed by one multiply by the float nearest
// to 1/sqrt(g).  Every add happens in that order on the GPU too, so the codes
// are bit-identical to a sequential evaluation of the same butterfly.
//
// Row kernel (small batches, weights, rows past 32768 elements; the
// token-block kernel below has its own layout): one workgroup of 256 threads
// per row.  A thread owns
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
// IEEE binary16 -> fp32 is exact (v_cvt_f32_f16)
__device__ inline float f16_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w)));
}
__device__ inline float f16_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}
// the two 16-bit input formats: bf16 bits (uint16_t) and IEEE binary16 (_Float16)
template <typename In> __device__ inline float in_lo(uint32_t w);
template <typename In> __device__ inline float in_hi(uint32_t w);
template <> __device__ inline float in_lo<uint16_t>(uint32_t w) { return bf16_lo(w); }
template <> __device__ inline float in_hi<uint16_t>(uint32_t w) { return bf16_hi(w); }
template <> __device__ inline float in_lo<_Float16>(uint32_t w) { return f16_lo(w); }
template <> __device__ inline float in_hi<_Float16>(uint32_t w) { return f16_hi(w); }

// Load 8 consecutive inputs as fp32.
template <typename In16>
__device__ inline void load8_16(const In16* p, float (&v)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  v[0] = in_lo<In16>(w.x); v[1] = in_hi<In16>(w.x);
  v[2] = in_lo<In16>(w.y); v[3] = in_hi<In16>(w.y);
  v[4] = in_lo<In16>(w.z); v[5] = in_hi<In16>(w.z);
  v[6] = in_lo<In16>(w.w); v[7] = in_hi<In16>(w.w);
}
__device__ inline void load8(const uint16_t* p, float (&v)[8]) { load8_16(p, v); }
__device__ inline void load8(const _Float16* p, float (&v)[8]) { load8_16(p, v); }
__device__ inline void load8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// v of lane (this lane ^ T).  Inside a 16-lane row DPP moves do it: xor 1
// and xor 2 are quad permutations, xor 4 is the quad reversal (xor 3)
// followed by the half-row mirror (xor 7), xor 8 is a rotation of the row by
// 8; wider distances go through ds_bpermute.
template <int T>
__device__ inline float lane_xor(float v) {
  const int b = __float_as_int(v);
  if constexpr (T == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0xB1, 0xF, 0xF, true));
  else if constexpr (T == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x4E, 0xF, 0xF, true));
  else if constexpr (T == 4)
    return __int_as_float(__builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(b, 0x1B, 0xF, 0xF, true), 0x141, 0xF, 0xF, true));
  else if constexpr (T == 8) return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x128, 0xF, 0xF, true));
  else return __shfl_xor(v, T);
}

// One butterfly stage between lanes T apart: the lower element keeps
// RN(a + b), the upper RN(a - b) (a = lower), each as RN(own * sgn + partner)
// with sgn = -1 on the upper lane.
template <int T>
__device__ inline void lane_stage(float (&v)[8], int lane_in_group) {
  const float sgn = (lane_in_group & T) != 0 ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = __builtin_fmaf(v[i], sgn, lane_xor<T>(v[i]));
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
  lane_stage<1>(v, lane_in_group);
  lane_stage<2>(v, lane_in_group);
  lane_stage<4>(v, lane_in_group);
  lane_stage<8>(v, lane_in_group);
  if constexpr (G == 256) lane_stage<16>(v, lane_in_group);
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

// Maximum over the workgroup (max is exact and order-free): inside each
// 16-lane row by DPP moves, over the four rows of a wave by lane reads, over
// the waves through LDS.
__device__ inline float block_max(float a) {
  __shared__ float part[kThreads / 64];
  a = fmaxf(a, lane_xor<1>(a));
  a = fmaxf(a, lane_xor<2>(a));
  a = fmaxf(a, lane_xor<4>(a));
  a = fmaxf(a, lane_xor<8>(a));
  a = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 0)),
                  __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 16))),
            fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 32)),
                  __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 48))));
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

// ---------------------------------------------------------------- token blocks
// Activation path for K <= 32768.  The workgroup's rows are staged through
// LDS by direct-to-LDS loads (each wave moves its own 32 blocks, 1 KB of
// consecutive input per instruction), and two lanes hold one 128-element
// block in registers: lane 2b + h takes elements [64h, 64h + 64) of block b.
// Stages h' = 1..32 stay in the lane; stage 64 pairs the two lanes (one DPP
// exchange); for g = 256 stage 128 pairs the same half of blocks b and b ^ 1
// (lanes two apart).  A lane that must keep a - b while it holds b computes
// RN(b - a) = -RN(a - b) with the same fma its partner uses for RN(a + b) and
// carries the sign into the final multiply (rounding to nearest is
// symmetric), so every add is the one the sequential butterfly does and the
// values match it up to the sign of an exact zero (a = b gives +0 where the
// butterfly has +0 too, turned into -0 by the negated constant), which neither
// the row maximum nor the code can see.  (The weight unpacking below, whose
// output is the values themselves, uses RN(own * sgn + partner) instead.)
// With
// 64 values per lane a wave needs about 94 registers, so twice as many waves
// share a SIMD as with a whole block per lane (4608 x 3072: 13.2 -> 11.7 us;
// 4608 x 12288: 43.5 -> 36.8 us; identical codes and scales).  The codes go
// back through LDS so that every wave stores its own blocks as 16-byte
// chunks of consecutive codes; the only workgroup barrier completes the
// per-row maxima (rows cross wave boundaries).
//
// Codes: rne(v / s) with the quotient correctly rounded, computed with a
// reciprocal and two fused multiply-adds instead of a full division per
// element (rows whose scale is too small for a normal reciprocal divide).
constexpr int kBlockElems = 128;
constexpr int kMaxBlocksPerWg = 256;                 // two lanes per block: 512 lanes
constexpr int kMaxBlockK = kMaxBlocksPerWg * kBlockElems;
constexpr int64_t kSmallBatchElems = int64_t{1} << 21;

// v[i] <- RN(v[i] + sgn * v[i] of the partner lane) for all 64 values, one
// v_fmac_f32 with a DPP source per value (the partner is the neighbour lane,
// P = 0, or the lane two away, P = 1, inside each quad).  Eight values per
// asm block; each block opens with the two wait states a DPP read needs after
// a VALU write of its source (inside a block no instruction reads what another
// of the block wrote).
template <int P>
__device__ inline void dpp_fmac8(float (&v)[64], float sgn) {
#define CONVROT_DPP8(i0, PERM)                                                                          \
  asm volatile("s_nop 1\n\t"                                                                            \
               "v_fmac_f32_dpp %0, %0, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"                      \
               "v_fmac_f32_dpp %1, %1, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"                      \
               "v_fmac_f32_dpp %2, %2, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"                      \
               "v_fmac_f32_dpp %3, %3, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"                      \
               "v_fmac_f32_dpp %4, %4, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"                      \
               "v_fmac_f32_dpp %5, %5, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"                      \
               "v_fmac_f32_dpp %6, %6, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"                      \
               "v_fmac_f32_dpp %7, %7, %8 " PERM " row_mask:0xf bank_mask:0xf"                            \
               : "+v"(v[i0]), "+v"(v[i0 + 1]), "+v"(v[i0 + 2]), "+v"(v[i0 + 3]), "+v"(v[i0 + 4]),         \
                 "+v"(v[i0 + 5]), "+v"(v[i0 + 6]), "+v"(v[i0 + 7])                                         \
               : "v"(sgn))
#pragma unroll
  for (int i = 0; i < 64; i += 8) {
    if constexpr (P == 0) CONVROT_DPP8(i, "quad_perm:[1,0,3,2]");
    else CONVROT_DPP8(i, "quad_perm:[2,3,0,1]");
  }
#undef CONVROT_DPP8
}

template <int G, typename In16>
__global__ __launch_bounds__(512) void rotq_block_kernel(
    const In16* __restrict__ x, int64_t M, int K, int rows_per_wg, uint32_t bpr_inv,
    int8_t* __restrict__ q, float* __restrict__ scale) {
  // the input tile, 256 bytes per block of the workgroup (sized at launch)
  extern __shared__ __attribute__((aligned(16))) uint4 tile[];
  __shared__ uint32_t row_amax[kMaxBlocksPerWg];
  const int tid = threadIdx.x;
  const int bpr = K / kBlockElems;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * rows_per_wg;
  const int rows = static_cast<int>(min(static_cast<int64_t>(rows_per_wg), M - row0));
  const int nblk = rows * bpr;

  if (tid < rows_per_wg) row_amax[tid] = 0u;
  __syncthreads();
  // wave w loads its own 32 blocks: instruction u fills LDS slots
  // p = 512 w + 64 u + lane, slot p holding chunk (p & 15) ^ (b & 15) of
  // block b = p >> 4
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wchunks = max(0, min(32, nblk - 32 * wave)) * 16;
  const char* wbase = reinterpret_cast<const char*>(x + row0 * K) + static_cast<int64_t>(wave) * 32 * 256;
  uint32_t loff[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    loff[r] = static_cast<uint32_t>(((lane >> 4) * 16 + ((lane & 15) ^ ((4 * r + (lane >> 4)) & 15))) * 16);
  if (wchunks == 512) {
    // a whole wave: eight unconditional loads, each a scalar base (kept
    // opaque, so that it stays in scalar registers) plus the lane's offset
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      asm volatile("" : "+v"(loff[u & 3]));
      const char* base = wbase + u * 1024;
      asm volatile("" : "+s"(base));
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(base + loff[u & 3]),
                                       (__attribute__((address_space(3))) void*)(tile + 512 * wave + 64 * u), 16, 0, 0);
    }
  } else {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u * 64 >= wchunks) break;
      if (64 * u + lane < wchunks) {
        asm volatile("" : "+v"(loff[u & 3]));
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(wbase + u * 1024 + loff[u & 3]),
                                         (__attribute__((address_space(3))) void*)(tile + 512 * wave + 64 * u), 16, 0, 0);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  const int b = tid >> 1, half = tid & 1;
  const bool active = b < nblk;
  // b / bpr as (b * bpr_inv) >> 16 with bpr_inv = ceil(2^16 / bpr), exact
  // for b < 256 and bpr <= 256 (checked for every pair), instead of an
  // integer division
  const int lrow = active ? static_cast<int>(__umul24(static_cast<uint32_t>(b), bpr_inv) >> 16) : 0;
  const bool row_first = b == lrow * bpr;
  float v[64];
  float amax = 0.0f;
  // the normalisation constant times the sign this lane's values carry
  float c = RotScale<G>::value;
  if (active) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const uint4 w = tile[b * 16 + ((8 * half + jj) ^ (b & 15))];
      v[8 * jj + 0] = in_lo<In16>(w.x); v[8 * jj + 1] = in_hi<In16>(w.x);
      v[8 * jj + 2] = in_lo<In16>(w.y); v[8 * jj + 3] = in_hi<In16>(w.y);
      v[8 * jj + 4] = in_lo<In16>(w.z); v[8 * jj + 5] = in_hi<In16>(w.z);
      v[8 * jj + 6] = in_lo<In16>(w.w); v[8 * jj + 7] = in_hi<In16>(w.w);
    }
#pragma unroll
    for (int h = 1; h < 64; h <<= 1) {
#pragma unroll
      for (int i = 0; i < 64; ++i) {
        if ((i & h) == 0) {
          const float a = v[i], d = v[i + h];
          v[i] = a + d;
          v[i + h] = a - d;
        }
      }
    }
    {  // stage 64: the lower half keeps RN(a + b), the upper RN(b - a)
      const float sgn = half ? -1.0f : 1.0f;
      c = half ? -c : c;
      dpp_fmac8<0>(v, sgn);
    }
    if constexpr (G == 256) {
      // stage 128: the same half of blocks b (even) and b ^ 1, two lanes
      // apart; both carry the same sign, so the odd block's RN(v - p)
      // flips it
      const bool odd = (b & 1) != 0;
      const float sgn = odd ? -1.0f : 1.0f;
      c = odd ? -c : c;
      dpp_fmac8<1>(v, sgn);
    }
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      v[i] = v[i] * c;
      amax = fmaxf(amax, fabsf(v[i]));
    }
    // one LDS atomic per block, or per two blocks when rows hold an even
    // number of blocks (a block pair then never straddles two rows): the
    // atomics of one row all hit one LDS word and are served one at a time
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(amax), 0xB1, 0xF, 0xF, false)));
    const bool pairs = (bpr & 1) == 0;
    if (pairs)
      amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(amax), 0x4E, 0xF, 0xF, false)));
    if ((tid & (pairs ? 3 : 1)) == 0)
      atomicMax(&row_amax[lrow], __float_as_uint(amax));   // amax >= 0: bit order = value order
  }
  __syncthreads();

  // codes -> LDS (block b's 8 code chunks at j ^ ((b >> 1) & 7); this lane
  // writes chunks 4 * half .. 4 * half + 3), then out
  uint4* codes = tile;
  if (active) {
    const float s = __uint_as_float(row_amax[lrow]) / 127.0f;
    if (row_first && half == 0) scale[row0 + lrow] = s;
    const float r = 1.0f / s;
    char* out = reinterpret_cast<char*>(codes) + b * 128;
    if (r < 1e30f) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        uint32_t wd[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          uint32_t t[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float val = v[16 * jj + 4 * d + e];
            const float q0 = val * r;
            const float rem = __builtin_fmaf(-q0, s, val);
            const float q1 = __builtin_fmaf(rem, r, q0);
            t[e] = __float_as_uint(q1 + 12582912.0f);
          }
          const uint32_t lo = __builtin_amdgcn_perm(t[1], t[0], 0x0c0c0400u);
          const uint32_t hi = __builtin_amdgcn_perm(t[3], t[2], 0x0c0c0400u);
          wd[d] = lo | (hi << 16);
        }
        reinterpret_cast<uint4*>(out)[(4 * half + jj) ^ ((b >> 1) & 7)] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      }
    } else {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        uint32_t wd[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          uint32_t packed = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            packed |= (static_cast<uint32_t>(quant_code(v[16 * jj + 4 * d + e], s)) & 0xffu) << (8 * e);
          wd[d] = s != 0.0f ? packed : 0u;
        }
        reinterpret_cast<uint4*>(out)[(4 * half + jj) ^ ((b >> 1) & 7)] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      }
    }
  }
  // this wave stores its own 32 blocks' codes
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  uint4* dstq = reinterpret_cast<uint4*>(q + row0 * K);
  const int wcodes = wchunks / 2;
  if (wcodes == 256) {
    // a whole wave: piece i of lane l is chunk l & 7 of block
    // 32 wave + (l >> 3) + 8 i, stored at chunk (l & 7) ^ (l >> 4) for even
    // i and ^ (l >> 4) ^ 4 for odd i: two lane offsets and immediates
    const char* cb = reinterpret_cast<const char*>(codes);
    const int o = (32 * wave + (lane >> 3)) * 128 + (((lane & 7) ^ (lane >> 4)) << 4);
    uint4* d = dstq + 256 * wave + lane;
#pragma unroll
    for (int i = 0; i < 4; ++i) d[64 * i] = *reinterpret_cast<const uint4*>(cb + (o ^ (64 * (i & 1))) + 1024 * i);
  } else {
    for (int cc = 256 * wave + lane; cc < 256 * wave + wcodes; cc += 64) {
      const int bb = cc >> 3, j = cc & 7;
      dstq[cc] = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(codes) + bb * 128)[j ^ ((bb >> 1) & 7)];
    }
  }
}

__global__ void zero_word_kernel(uint32_t* p) { *p = 0u; }

// ---------------------------------------------------------------- default path
// Unpacking of a rotated int8 weight for the default (dequantizing) path
// (page "int8 Compute", "What stays on the default path": such layers keep
// unpacking their weights): every row is dequantized (s * q in fp32) and
// rotated back by R, which is its own inverse (symmetric and orthogonal), so
// the same butterfly in the same order applies; the result is rounded to
// bf16 or fp16.  Two lanes per 128-element block, as in the token-block
// kernel: lane 2b + h dequantizes and rotates elements [64h, 64h + 64) of
// block b (blocks counted over the whole row-major weight), stages 1..32 in
// the lane, stage 64 by one DPP exchange, stage 128 (g = 256) with the same
// half of block b ^ 1.  Both lanes of an exchange run RN(own * sgn + partner),
// sgn = +1 where a + b is kept and -1 where the lane holds b and keeps a - b,
// so every value, zeros' signs included, is the sequential butterfly's.  No
// LDS and no barrier: every lane reads 64 contiguous codes and writes 128
// contiguous bytes (12288 x 3072: 30-33 us like the one-row-per-workgroup
// kernel it replaced at g = 128, 30 instead of 35 us at g = 256).
template <int G, bool OutF16>
__global__ __launch_bounds__(256) void unpack_block_kernel(
    const int8_t* __restrict__ wq, int64_t nblk, int bpr, const float* __restrict__ w_scale, int row_scale,
    uint16_t* __restrict__ out) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t b = t >> 1;
  const int half = static_cast<int>(t & 1);
  // whole blocks (and, for g = 256, whole block pairs: rows hold an even
  // number of blocks) leave together, so every exchange partner is active
  if (b >= nblk) return;
  const float s = w_scale[row_scale ? b / bpr : 0];
  const uint4* src = reinterpret_cast<const uint4*>(wq + b * 128 + 64 * half);
  float v[64];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 w = src[c];
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[16 * c + 4 * k + i] = s * static_cast<float>(static_cast<int8_t>(wd[k] >> (8 * i)));
  }
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], d = v[i + h];
        v[i] = a + d;
        v[i + h] = a - d;
      }
    }
  }
  {  // stage 64: the lower lane keeps RN(a + b), the upper RN(a - b)
    const float sgn = half ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const float p = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v[i]), 0xB1, 0xF, 0xF, false));
      v[i] = __builtin_fmaf(v[i], sgn, p);
    }
  }
  if constexpr (G == 256) {  // stage 128: block b (even) keeps RN(a + b), b ^ 1 RN(a - b)
    const float sgn = (b & 1) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const float p = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v[i]), 0x4E, 0xF, 0xF, false));
      v[i] = __builtin_fmaf(v[i], sgn, p);
    }
  }
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    v[i] = v[i] * RotScale<G>::value;
    // fp16 output: keep the product in fp32 (no fused multiply + conversion)
    if constexpr (OutF16) asm volatile("" : "+v"(v[i]));
  }
  uint4* dst = reinterpret_cast<uint4*>(out + b * 128 + 64 * half);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t lo, hi;
      if constexpr (OutF16) {
        lo = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v[8 * j + 2 * i]));
        hi = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v[8 * j + 2 * i + 1]));
      } else {
        lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[8 * j + 2 * i]));
        hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[8 * j + 2 * i + 1]));
      }
      p[i] = static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
    }
    dst[j] = make_uint4(p[0], p[1], p[2], p[3]);
  }
}

template <int G, bool OutF16>
hipError_t launch_unpack_g(const int8_t* wq, const float* w_scale, bool row_scale, int64_t N, int64_t K,
                           uint16_t* out, hipStream_t stream) {
  const int64_t nblk = N * (K / 128);
  const int64_t wgs = (2 * nblk + 255) / 256;
  hipLaunchKernelGGL((unpack_block_kernel<G, OutF16>), dim3(static_cast<uint32_t>(wgs)), dim3(256), 0, stream, wq,
                     nblk, static_cast<int>(K / 128), w_scale, row_scale ? 1 : 0, out);
  return hipGetLastError();
}

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

namespace {

template <typename In16>
hipError_t rotate_quant_16(const In16* x, int64_t M, int64_t K, int group, int8_t* q,
                           float* scale, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  // Small batches (up to 2^21 elements, e.g. 512 x 4096) with rows shorter
  // than 8192: the token-block kernel has only a handful of waves there, and
  // the row kernel, which spreads a row over 256 lanes, is faster (16 x 4096:
  // 3.2 us instead of 5.4; 256 x 3072: 3.4 instead of 5.4).  From K = 8192 on
  // a row kernel lane holds four or more chunks in a serial chain, and the
  // block kernel wins at any batch (16 x 12288: 5.7 us instead of 8.1;
  // 16 x 16384, rotated twice by the row kernel: 5.8 instead of 16.1).
  if (K <= kMaxBlockK && (M * K > kSmallBatchElems || K >= 8192)) {
    // Rows per workgroup: as many as fit (256 blocks, 512 lanes), but no more
    // than an even share of two workgroups per CU, so that every CU gets the
    // same work when the batch is small (M = 4608, K = 3072: 512 workgroups of
    // 9 rows instead of 461 of 10, of which 205 CUs would run two).  Where
    // that share is two rows, one row per workgroup is taken when it puts
    // fewer rows on the busiest CU (M = 701, K = 3072: 701 workgroups, at
    // most 3 rows per CU instead of 4; 5.7 us instead of 6.7).  Two lanes
    // per block, threads rounded up to whole waves; LDS holds 256 bytes per
    // block, sized at launch (K = 12288: 48 KB, three workgroups per CU).
    const int fit = kMaxBlocksPerWg / static_cast<int>(K / kBlockElems);
    const int64_t cus = num_cus();
    int64_t share = (M + 2 * cus - 1) / (2 * cus);
    if (share == 2 && (M + cus - 1) / cus < 2 * (((M + 1) / 2 + cus - 1) / cus)) share = 1;
    const int rows_per_wg = static_cast<int>(share < fit ? share : fit);
    const int64_t wgs = (M + rows_per_wg - 1) / rows_per_wg;
    const int blocks = rows_per_wg * static_cast<int>(K / kBlockElems);
    const int threads = (2 * blocks + 63) / 64 * 64;
    const size_t lds = static_cast<size_t>(blocks) * 256;
    const uint32_t bpr = static_cast<uint32_t>(K / kBlockElems);
    const uint32_t bpr_inv = (65536u + bpr - 1u) / bpr;
    if (group == 128)
      hipLaunchKernelGGL((rotq_block_kernel<128, In16>), dim3(static_cast<uint32_t>(wgs)), dim3(threads), lds,
                         stream, x, M, static_cast<int>(K), rows_per_wg, bpr_inv, q, scale);
    else
      hipLaunchKernelGGL((rotq_block_kernel<256, In16>), dim3(static_cast<uint32_t>(wgs)), dim3(threads), lds,
                         stream, x, M, static_cast<int>(K), rows_per_wg, bpr_inv, q, scale);
    return hipGetLastError();
  }
  return dispatch_group<In16, kActQuant>(group, x, M, K, q, scale, nullptr, stream);
}

}  // namespace

int num_cus() {
  // read once (thread-safe static initialisation), from the device current
  // at the first call
  static const int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      return v;
    return 256;
  }();
  return n;
}

hipError_t launch_unpack_weight(const int8_t* wq, const float* w_scale, bool row_scale, int64_t N,
                                int64_t K, int group, bool out_f16, uint16_t* out, hipStream_t stream) {
  if (group == 128)
    return out_f16 ? launch_unpack_g<128, true>(wq, w_scale, row_scale, N, K, out, stream)
                   : launch_unpack_g<128, false>(wq, w_scale, row_scale, N, K, out, stream);
  return out_f16 ? launch_unpack_g<256, true>(wq, w_scale, row_scale, N, K, out, stream)
                 : launch_unpack_g<256, false>(wq, w_scale, row_scale, N, K, out, stream);
}

hipError_t launch_rotate_quant(const uint16_t* x, int64_t M, int64_t K, int group, int8_t* q,
                               float* scale, hipStream_t stream) {
  return rotate_quant_16(x, M, K, group, q, scale, stream);
}

hipError_t launch_rotate_quant_f16(const uint16_t* x, int64_t M, int64_t K, int group, int8_t* q,
                                   float* scale, hipStream_t stream) {
  return rotate_quant_16(reinterpret_cast<const _Float16*>(x), M, K, group, q, scale, stream);
}

hipError_t launch_prepare_weight(const void* w, int in_dtype, bool row_scale, int64_t N, int64_t K,
                                 int group, int8_t* wq, float* w_scale, uint32_t* amax_cell,
                                 hipStream_t stream) {
  // One scale per output channel: every weight row is quantized exactly like
  // a token (the same rotation, absmax, scale and codes).
  if (row_scale) {
    if (in_dtype == kInBf16)
      return rotate_quant_16(static_cast<const uint16_t*>(w), N, K, group, wq, w_scale, stream);
    if (in_dtype == kInF16)
      return rotate_quant_16(static_cast<const _Float16*>(w), N, K, group, wq, w_scale, stream);
    return dispatch_group<float, kActQuant>(group, static_cast<const float*>(w), N, K, wq, w_scale,
                                            nullptr, stream);
  }
  hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(1), 0, stream, amax_cell);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (in_dtype == kInBf16) {
    const auto* x = static_cast<const uint16_t*>(w);
    e = dispatch_group<uint16_t, kWeightAbsmax>(group, x, N, K, nullptr, nullptr, amax_cell, stream);
    if (e != hipSuccess) return e;
    return dispatch_group<uint16_t, kWeightQuant>(group, x, N, K, wq, w_scale, amax_cell, stream);
  }
  if (in_dtype == kInF16) {
    const auto* x = static_cast<const _Float16*>(w);
    e = dispatch_group<_Float16, kWeightAbsmax>(group, x, N, K, nullptr, nullptr, amax_cell, stream);
    if (e != hipSuccess) return e;
    return dispatch_group<_Float16, kWeightQuant>(group, x, N, K, wq, w_scale, amax_cell, stream);
  }
  const auto* x = static_cast<const float*>(w);
  e = dispatch_group<float, kWeightAbsmax>(group, x, N, K, nullptr, nullptr, amax_cell, stream);
  if (e != hipSuccess) return e;
  return dispatch_group<float, kWeightQuant>(group, x, N, K, wq, w_scale, amax_cell, stream);
}

}  // namespace convrot
